"""Plain, slow fp64 CPU oracle for the AKV cache-engineering hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, tables or
helpers with the HIP library; both sides only consume the seeded inputs made
by ``agent_kv_cache_amd.workloads``.

Sources (cited by page title and section, never by line):

* [CE]  review of "Cache Engineering for Agents" (Tianyu Fu et al.),
        euisuk-chung.github.io, 2026-10-29 -- section 3.3 defines the three
        cache operations (eqs. 3-5), section 3.4 the operation sequence
        (eq. 6), Appendix A.1.1 / Figure 10 walks positions through a
        drop / reposition history.
* [AKV] "[Repo Review] AKV" (thu-nics/AKV static review),
        euisuk-chung.github.io, 2026-10-23 -- section 1 (drop before
        reposition at one boundary), section 1.1 (the five-message worked
        example), section 5.5 (the reposition kernel: FP32 un-rotate then
        rotate, equal positions are copied, V is copied, not rotated).

What is computed (every function below is the plain definition):

* append (eq. 3):  new entries are concatenated after the active ones and
  take positions next_pos, next_pos+1, ...; next_pos advances.  The model
  rotates the new keys at those positions; append_rotated does that step
  here (one fp64 rotation, one rounding).  release empties a sequence and
  resets its next position (a request ends; its pages return to the pool).
* drop (eq. 4):    an order-preserving removal of the active entries named by
  an index set.  Survivors keep their order, K, V, positions and token id;
  next_pos is NOT lowered.
* repos (eq. 5):   K' = R(q) R(p)^-1 K for each survivor, with R the NeoX
  half-split RoPE rotation (pair i = (k[i], k[i + d/2]) rotated by
  +pos * theta_i, theta_i = base^(-2i/d)).  R(q) R(p)^-1 = R(q - p), so one
  angle (q - p) * theta_i per pair.  The canonical target is q = 0..r-1 and
  next_pos becomes r.  V is never touched.  Delta = 0 leaves K bit-identical.
* decode attention: softmax(q K^T / sqrt(d)) V over the first active_len
  entries, GQA head h reads kv head floor(h / G).
* replay (eq. 6):  the state is the result of applying the op list in order
  from the empty cache.
* fork ([CE] sec. 4.2.3, Appendix A.1.1): a new position version of a
  sequence -- its entries copied (K re-rotated when positions change, V
  copied), then drop / reposition applied to the copy only; the source
  version is unchanged.
* segment attention ([CE] Appendix A.1.1): a restore forward splits its
  queries into segments; each segment applies standard causal attention over
  its own KV list, whose last n entries are the segment's own tokens.

* RoPE variants ([AKV] sec. 5.5): partial RoPE rotates only the first
  rotary_dim dimensions (pairs (i, i + rotary_dim/2)) and copies the rest of
  K; sliding-window layers read, per query, the entries whose position lies
  in the window (positions, not indices, after a drop); frequencies may be
  replaced by a caller table (Llama 3.1 / YaRN rules below, not on the pages).

Readings where the pages are silent:
  pairing/sign of RoPE (NeoX half split, +p*theta), theta_i without scaling,
  one fp64 rounding to bf16 (round half to even) per rotated element, no
  self-token and no sinks in decode, scale 1/sqrt(d), 1 = drop in masks.

All arithmetic is numpy float64.  K and V are held as float64 arrays whose
values are exactly representable in bfloat16.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

__all__ = [
    "BF16_MAX",
    "bf16_round",
    "bf16_bits",
    "bf16_from_bits",
    "bf16_ulp_distance",
    "rope_theta",
    "llama3_theta",
    "yarn_theta",
    "rotate_pairs",
    "rerotate_keys",
    "attend",
    "SeqState",
    "OracleCache",
    "segment_attention",
    "replay",
]

# Largest finite bfloat16: fraction 1.1111111b, exponent 127.
BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


# ---------------------------------------------------------------------------
# bfloat16 from its definition
# ---------------------------------------------------------------------------
def bf16_round(x) -> np.ndarray:
    """Round float64 values to bfloat16 in ONE step, ties to even.

    bfloat16 keeps 8 significant bits (1 implicit + 7 stored) and float32's
    exponent range.  For |x| in [2^(e-1), 2^e) the spacing is 2^(e-8);
    below the smallest normal (2^-126) the spacing is fixed at 2^-133.
    Values whose rounded magnitude exceeds BF16_MAX become +-inf.  The sign of
    zero is kept (rint keeps it).  No float32 intermediate is used, so there
    is no double rounding.
    """
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    fin = np.isfinite(x)
    xf = x[fin]
    _, e = np.frexp(xf)                       # |xf| in [2^(e-1), 2^e)
    q = np.maximum(e - 8, -133)               # exponent of the spacing
    y = np.ldexp(np.rint(np.ldexp(xf, -q)), q)  # power-of-two scalings are exact
    over = np.abs(y) > BF16_MAX
    y[over] = np.copysign(np.inf, xf[over])
    out[fin] = y
    return out


def bf16_bits(x) -> np.ndarray:
    """uint16 bit patterns of float64 values that are already bf16 values."""
    x = np.asarray(x, dtype=np.float64)
    f = x.astype(np.float32)                  # exact: bf16 values fit in fp32
    if not np.array_equal(f.astype(np.float64), x, equal_nan=True):
        raise ValueError("bf16_bits: input is not bf16-representable")
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def bf16_from_bits(u) -> np.ndarray:
    """float64 values of uint16 bfloat16 bit patterns (bits are the top half of fp32)."""
    u = np.asarray(u, dtype=np.uint16)
    with np.errstate(invalid="ignore"):          # NaN payloads convert quietly
        return (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_ulp_distance(a_bits, b_bits) -> np.ndarray:
    """Number of bf16 steps between two bit patterns (+0 and -0 coincide)."""
    def ordered(u):
        u = np.asarray(u, dtype=np.uint16).astype(np.int64)
        mag = u & 0x7FFF
        return np.where(u & 0x8000, -mag, mag)
    return np.abs(ordered(a_bits) - ordered(b_bits))


# ---------------------------------------------------------------------------
# RoPE re-rotation ([CE] sec. 3.3, eq. 5; [AKV] sec. 5.5)
# ---------------------------------------------------------------------------
def rope_theta(head_dim: int, base: float, rotary_dim: Optional[int] = None) -> np.ndarray:
    """theta_i = base^(-2i/r) for i in [0, r/2), float64, no frequency scaling.

    r = rotary_dim (default head_dim).  With partial RoPE only the first r
    dimensions of a head are rotated ([AKV] sec. 5.5: the rest of K is copied).
    """
    r = head_dim if rotary_dim is None else int(rotary_dim)
    if r % 2 or not 0 < r <= head_dim:
        raise ValueError("rotary_dim must be even and in (0, head_dim]")
    i = np.arange(r // 2, dtype=np.float64)
    return np.power(np.float64(base), -2.0 * i / r)


def llama3_theta(theta: np.ndarray, factor: float, low_freq_factor: float,
                 high_freq_factor: float, original_max_pos: int) -> np.ndarray:
    """Frequencies of the Llama 3.1 RoPE scaling rule applied to theta.

    Not on the pages: the published rule of the Llama 3.1 release, written
    here from its definition.  With wavelength w = 2 pi / theta and the
    original context length C: w < C / high_freq_factor keeps theta;
    w > C / low_freq_factor divides it by factor; in between it blends
    linearly in C / w: s = (C / w - low) / (high - low),
    theta' = (1 - s) theta / factor + s theta.
    """
    theta = np.asarray(theta, dtype=np.float64)
    w = 2.0 * np.pi / theta
    lo_w = original_max_pos / low_freq_factor
    hi_w = original_max_pos / high_freq_factor
    s = (original_max_pos / w - low_freq_factor) / (high_freq_factor - low_freq_factor)
    mid = (1.0 - s) * theta / factor + s * theta
    return np.where(w < hi_w, theta, np.where(w > lo_w, theta / factor, mid))


def yarn_theta(rotary_dim: int, base: float, factor: float, original_max_pos: int,
               beta_fast: float = 32.0, beta_slow: float = 1.0) -> np.ndarray:
    """Frequencies of YaRN's "NTK-by-parts" interpolation.

    Not on the pages: the published method (Peng et al., 2023), written here
    from its definition.  Dimension pair i turns original_max_pos * theta_i /
    (2 pi) times over the original context; pairs that turn more than
    beta_fast times keep theta_i, pairs that turn fewer than beta_slow times
    use theta_i / factor, and a linear ramp in i joins the two.  The ramp ends
    are the (real) pair indices where the turn count equals beta_fast and
    beta_slow, floored and ceiled, clamped to [0, r - 1].  YaRN's attention
    temperature scales cos and sin of every position alike, so it does not
    enter a re-rotation R(q - p).
    """
    r = int(rotary_dim)
    theta = rope_theta(r, base)

    def pair_at(turns):
        return r * np.log(original_max_pos / (turns * 2.0 * np.pi)) / (2.0 * np.log(base))

    lo = max(int(np.floor(pair_at(beta_fast))), 0)
    hi = min(int(np.ceil(pair_at(beta_slow))), r - 1)
    if lo == hi:
        hi = lo + 1e-3
    i = np.arange(r // 2, dtype=np.float64)
    ramp = np.clip((i - lo) / (hi - lo), 0.0, 1.0)      # 0: keep, 1: interpolate
    return theta * (1.0 - ramp) + (theta / factor) * ramp


def rotate_pairs(k: np.ndarray, delta, theta: np.ndarray) -> np.ndarray:
    """Unrounded fp64 NeoX rotation of the last axis by delta * theta_i.

    k: [..., d].  delta: int array broadcastable to k.shape[:-1] (typically
    one value per token, shape [n, 1, 1] against k [n, L, H, d]).
    The rotary part is the first r = 2 * len(theta) dimensions (r = d for
    full RoPE).  Pair i is (k[..., i], k[..., i + r/2]); it turns by the angle
    delta * theta_i (one fp64 product of the exact integer and theta_i):
        x' = x cos - y sin,   y' = y cos + x sin.
    Dimensions [r, d) are returned unchanged ([AKV] sec. 5.5).
    """
    k = np.asarray(k, dtype=np.float64)
    half = np.asarray(theta).shape[-1]
    r = 2 * half
    if r > k.shape[-1]:
        raise ValueError("rotate_pairs: more frequencies than dimension pairs")
    d = np.asarray(delta, dtype=np.float64)[..., None]      # [..., 1]
    ang = d * theta                                           # [..., r/2]
    c, s = np.cos(ang), np.sin(ang)
    x, y = k[..., :half], k[..., half:r]
    xr, yr = x * c - y * s, y * c + x * s
    tail = np.broadcast_to(k[..., r:], xr.shape[:-1] + (k.shape[-1] - r,))
    return np.concatenate([xr, yr, tail], axis=-1)


def rerotate_keys(k: np.ndarray, delta: np.ndarray, theta: np.ndarray) -> np.ndarray:
    """K' = bf16(R(delta) K) per token; tokens with delta == 0 are returned unchanged.

    k: [n, L, H, d] bf16 values in float64; delta: [n] integers.
    """
    k = np.asarray(k, dtype=np.float64)
    delta = np.asarray(delta, dtype=np.int64)
    out = k.copy()
    moved = np.flatnonzero(delta != 0)
    if moved.size:
        dd = delta[moved].reshape((-1,) + (1,) * (k.ndim - 2))
        out[moved] = bf16_round(rotate_pairs(k[moved], dd, theta))
    return out


# ---------------------------------------------------------------------------
# Decode attention
# ---------------------------------------------------------------------------
def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Softmax attention of one query row over n keys, fp64.

    q: [d], k: [n, d], v: [n, d].  s_j = q.k_j / sqrt(d); weights are
    exp(s - max s) normalised; output sum_j w_j v_j.  n == 0 gives zeros.
    """
    q = np.asarray(q, dtype=np.float64)
    n = k.shape[0]
    if n == 0:
        return np.zeros(q.shape[-1], dtype=np.float64)
    s = (k @ q) / np.sqrt(np.float64(q.shape[-1]))
    w = np.exp(s - s.max())
    w /= w.sum()
    return w @ v


# ---------------------------------------------------------------------------
# Cache state
# ---------------------------------------------------------------------------
@dataclass
class SeqState:
    """Active entries of one sequence in logical order, plus next_pos."""
    token_ids: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int64))
    pos: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int64))
    k: Optional[np.ndarray] = None      # [n, L, Hkv, d] float64 (bf16 values)
    v: Optional[np.ndarray] = None
    next_pos: int = 0

    def __len__(self) -> int:
        return int(self.token_ids.shape[0])


class OracleCache:
    """Per-sequence ordered lists of (token id, position, K, V) and next_pos.

    With ``with_kv=False`` only token ids and positions are tracked, which is
    enough to replay indices and positions of long histories.
    """

    def __init__(self, n_layers: int, n_kv_heads: int, head_dim: int,
                 rope_base: float, n_seqs: int = 1, with_kv: bool = True,
                 rotary_dim: Optional[int] = None, theta: Optional[np.ndarray] = None,
                 window: Optional[Sequence[int]] = None):
        """rotary_dim: partial RoPE (first rotary_dim dims rotated, default
        head_dim); theta: explicit frequencies (rotary_dim / 2 values, e.g.
        from llama3_theta / yarn_theta) instead of base^(-2i/r); window: per
        layer sliding-window length (0 or None = full attention)."""
        if head_dim % 2:
            raise ValueError("head_dim must be even for half-split RoPE")
        self.n_layers, self.n_kv_heads, self.head_dim = n_layers, n_kv_heads, head_dim
        r = head_dim if rotary_dim is None else int(rotary_dim)
        if theta is None:
            self.theta = rope_theta(head_dim, rope_base, r)
        else:
            self.theta = np.asarray(theta, dtype=np.float64).reshape(-1)
            if 2 * self.theta.shape[0] != r:
                raise ValueError("theta needs rotary_dim / 2 values")
        self.rotary_dim = r
        self.window = [0] * n_layers if window is None else [int(w or 0) for w in window]
        if len(self.window) != n_layers or min(self.window) < 0:
            raise ValueError("window needs one value >= 0 per layer")
        self.with_kv = with_kv
        shape = (0, n_layers, n_kv_heads, head_dim)
        self.seqs: List[SeqState] = [
            SeqState(k=np.zeros(shape) if with_kv else None,
                     v=np.zeros(shape) if with_kv else None)
            for _ in range(n_seqs)
        ]

    # -- eq. (3): append --------------------------------------------------
    def append(self, b: int, token_ids, k=None, v=None) -> None:
        """Concatenate n entries at positions next_pos .. next_pos+n-1 ([CE] eq. 3).

        K must already be rotated at those positions (the model computes it);
        K and V are taken as given bf16 values.
        """
        s = self.seqs[b]
        tid = np.asarray(token_ids, dtype=np.int64).reshape(-1)
        n = tid.shape[0]
        s.token_ids = np.concatenate([s.token_ids, tid])
        s.pos = np.concatenate([s.pos, s.next_pos + np.arange(n, dtype=np.int64)])
        s.next_pos += n
        if self.with_kv:
            k = np.asarray(k, dtype=np.float64)
            v = np.asarray(v, dtype=np.float64)
            want = (n, self.n_layers, self.n_kv_heads, self.head_dim)
            if k.shape != want or v.shape != want:
                raise ValueError(f"append: K/V shape must be {want}")
            s.k = np.concatenate([s.k, k])
            s.v = np.concatenate([s.v, v])

    def append_rotated(self, b: int, token_ids, k_raw, v) -> None:
        """Append with the model's RoPE applied here (the rotation step of
        eq. 3 fused into the append): entry j takes position p_j = next_pos + j
        and key bf16(R(p_j) k_raw_j) -- one fp64 rotation by p_j * theta_i,
        rounded once; V is stored as given.  k_raw: [n, L, H, d] bf16 values.
        """
        s = self.seqs[b]
        k_raw = np.asarray(k_raw, dtype=np.float64)
        n = k_raw.shape[0]
        pos = (s.next_pos + np.arange(n, dtype=np.int64)).reshape((n,) + (1,) * (k_raw.ndim - 2))
        self.append(b, token_ids, bf16_round(rotate_pairs(k_raw, pos, self.theta)), v)

    def release(self, b: int) -> None:
        """End of a request: the sequence becomes empty and its next position
        returns to 0 (its pages go back to the free pool)."""
        shape = (0, self.n_layers, self.n_kv_heads, self.head_dim)
        self.seqs[b] = SeqState(k=np.zeros(shape) if self.with_kv else None,
                                v=np.zeros(shape) if self.with_kv else None)

    # -- eq. (4): drop ----------------------------------------------------
    def drop(self, b: int, mask) -> np.ndarray:
        """Remove the entries whose mask is 1, keeping order ([CE] eq. 4).

        Returns src: src[j] = pre-drop index of the j-th survivor.
        Positions, K, V and next_pos are untouched.
        """
        s = self.seqs[b]
        mask = np.asarray(mask).astype(bool).reshape(-1)
        if mask.shape[0] != len(s):
            raise ValueError("drop: mask length must equal the active length")
        src = np.flatnonzero(~mask)
        s.token_ids = s.token_ids[src]
        s.pos = s.pos[src]
        if self.with_kv:
            s.k = s.k[src]
            s.v = s.v[src]
        return src

    # -- eq. (5): reposition ----------------------------------------------
    def reposition(self, b: int, new_pos=None) -> np.ndarray:
        """Move every entry from its position p to q, K' = R(q - p) K ([CE] eq. 5).

        new_pos=None means the canonical 0..r-1.  new_pos must be >= 0 and
        strictly increasing.  next_pos becomes last(new_pos) + 1 (r for the
        canonical target, 0 when the cache is empty).  Returns delta = q - p.
        """
        s = self.seqs[b]
        r = len(s)
        q = (np.arange(r, dtype=np.int64) if new_pos is None
             else np.asarray(new_pos, dtype=np.int64).reshape(-1))
        if q.shape[0] != r:
            raise ValueError("reposition: new_pos length must equal the active length")
        if r and (q[0] < 0 or np.any(np.diff(q) <= 0)):
            raise ValueError("reposition: new_pos must be >= 0 and strictly increasing")
        delta = q - s.pos
        if self.with_kv:
            s.k = rerotate_keys(s.k, delta, self.theta)
        s.pos = q
        s.next_pos = int(q[-1]) + 1 if r else 0
        return delta

    def drop_reposition(self, b: int, mask, new_pos=None):
        """Drop, then reposition, at one boundary ([AKV] sec. 1: drop runs first)."""
        src = self.drop(b, mask)
        delta = self.reposition(b, new_pos)
        return src, delta

    # -- position versions ([CE] sec. 4.2.3, A.1.1) ------------------------
    def fork(self, src: int, dst: int, mask=None, reposition: bool = False, new_pos=None):
        """dst (empty) becomes a copy of src; then drop(mask) and, if asked,
        reposition(new_pos) are applied to dst only.  src is unchanged."""
        s, d = self.seqs[src], self.seqs[dst]
        if len(d) or src == dst:
            raise ValueError("fork: destination must be empty and differ from the source")
        d.token_ids = s.token_ids.copy()
        d.pos = s.pos.copy()
        d.next_pos = s.next_pos
        if self.with_kv:
            d.k = s.k.copy()
            d.v = s.v.copy()
        if mask is not None:
            self.drop(dst, mask)
        if reposition:
            self.reposition(dst, new_pos)

    # -- decode attention over the active KV ------------------------------
    def visible(self, b: int, upto: int, qpos: int, layer: int) -> np.ndarray:
        """Indices a query at position qpos sees among the first `upto` entries.

        Full attention: all of them.  Sliding window W ([AKV] sec. 5.5, the
        attention plan): the entries whose *position* is at least
        qpos - W + 1.  After a drop without reposition positions have gaps,
        so the window is not the last W indices.
        """
        idx = np.arange(upto)
        w = self.window[layer]
        if w:
            idx = idx[self.seqs[b].pos[:upto] >= qpos - w + 1]
        return idx

    def decode_attention(self, b: int, q, active_len: Optional[int] = None) -> np.ndarray:
        """o[l, h] = attend(q[l, h], K[vis, l, h // G], V[vis, l, h // G]).

        q: [L, Hq, d] (bf16 values).  vis = the first active_len entries
        (default: all), cut by the layer's sliding window for a query at
        position next_pos (the token being decoded).
        """
        s = self.seqs[b]
        q = np.asarray(q, dtype=np.float64)
        n = len(s) if active_len is None else int(active_len)
        if not 0 <= n <= len(s):
            raise ValueError("decode_attention: active_len out of range")
        L, Hq, d = q.shape
        G = Hq // self.n_kv_heads
        out = np.zeros((L, Hq, d))
        for l in range(L):
            vis = self.visible(b, n, s.next_pos, l)
            rng = _contiguous_range(vis)
            for g in range(self.n_kv_heads):
                if rng is None:
                    k, v = s.k[vis, l, g], s.v[vis, l, g]
                else:
                    k = np.ascontiguousarray(s.k[rng[0]:rng[1], l, g])
                    v = np.ascontiguousarray(s.v[rng[0]:rng[1], l, g])
                for h in range(g * G, (g + 1) * G):
                    out[l, h] = attend(q[l, h], k, v)
        return out


def _contiguous_range(vis: np.ndarray):
    """(a, z) when the index set `vis` is the range [a, z), else None.  A
    visible set always is one (positions strictly increase, so a window keeps
    a suffix of the prefix); rows are then sliced, not gathered row by row --
    the same values in the same order."""
    if vis.size == 0:
        return 0, 0
    a, z = int(vis[0]), int(vis[-1]) + 1
    return (a, z) if z - a == vis.size else None


def segment_attention(cache: "OracleCache", segments) -> list:
    """Causal attention of restore segments ([CE] Appendix A.1.1).

    segments: list of (b, q) with q [n, L, Hq, d]: the n query rows are the
    last n entries of sequence b (the segment's own tokens); row i attends to
    entries [0, len_b - n + i], cut by the layer's sliding window for a query
    at that row's own position.  Returns one [n, L, Hq, d] array per segment.
    """
    out = []
    for b, q in segments:
        q = np.asarray(q, dtype=np.float64)
        n = q.shape[0]
        s = cache.seqs[b]
        if n > len(s):
            raise ValueError("segment_attention: more queries than entries")
        L, Hq, d = q.shape[1:]
        G = Hq // cache.n_kv_heads
        o = np.zeros_like(q)
        for l in range(L):
            for g in range(cache.n_kv_heads):
                kc = np.ascontiguousarray(s.k[:, l, g])     # [len, d], one copy per head
                vc = np.ascontiguousarray(s.v[:, l, g])
                for i in range(n):
                    me = len(s) - n + i                       # this row's own entry
                    vis = cache.visible(b, me + 1, int(s.pos[me]), l)
                    rng = _contiguous_range(vis)
                    k, v = (kc[vis], vc[vis]) if rng is None else (kc[rng[0]:rng[1]],
                                                                   vc[rng[0]:rng[1]])
                    for h in range(g * G, (g + 1) * G):
                        o[i, l, h] = attend(q[i, l, h], k, v)
        out.append(o)
    return out


# ---------------------------------------------------------------------------
# eq. (6): replay of an operation history
# ---------------------------------------------------------------------------
def replay(cache: OracleCache, history: Sequence[tuple]) -> OracleCache:
    """Apply ops in order ([CE] sec. 3.4, eq. 6).

    Each op is a tuple whose first item names it:
      ("append", b, token_ids[, k, v])
      ("drop", b, mask)
      ("repos", b, new_pos_or_None)
      ("drop_repos", b, mask, new_pos_or_None)
    """
    for op in history:
        kind, b = op[0], op[1]
        if kind == "append":
            cache.append(b, op[2], *(op[3:5] if len(op) > 3 else (None, None)))
        elif kind == "drop":
            cache.drop(b, op[2])
        elif kind == "repos":
            cache.reposition(b, op[2])
        elif kind == "drop_repos":
            cache.drop_reposition(b, op[2], op[3])
        else:
            raise ValueError(f"replay: unknown op {kind!r}")
    return cache
