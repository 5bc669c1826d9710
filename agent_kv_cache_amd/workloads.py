"""Seeded synthetic inputs shaped like the pages' agent workloads.

This module holds NO arithmetic of the method (no rotation, no compaction, no
attention).  It only draws structure (sequence lengths, dropped tool-response
spans, block orders, the operation history of a long agent run) and bf16
~N(0,1) tensors.  Both the HIP path and the CPU oracle consume what it makes.

A rotated isotropic Gaussian is again an isotropic Gaussian, so keys that are
"pre-rotated by RoPE at their positions" have exactly the distribution of
plain N(0,1) draws; the generator therefore draws them directly.

Structure seeds use numpy PCG64; tensor data uses torch generators (CPU for
small cases, the GPU generator for the full-size cases).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

BLOCK = 16          # tokens per KV page


@dataclass(frozen=True)
class Shape:
    n_layers: int
    n_kv_heads: int
    head_dim: int
    n_q_heads: int
    rope_base: float

    @property
    def kv_bytes_per_token(self) -> int:
        """K+V bf16 bytes of one token over all layers and kv heads."""
        return self.n_layers * self.n_kv_heads * self.head_dim * 2 * 2


@dataclass
class Workload:
    """One drop+reposition then decode step over a batch of sequences."""
    name: str
    shape: Shape
    seq_lens: List[int]
    masks: List[np.ndarray]               # u8 per sequence, 1 = drop
    block_order: Optional[np.ndarray]     # None = in-order pages, else a permutation
    data_seed: int
    description: str = ""
    spans: List[List[Tuple[int, int]]] = field(default_factory=list)

    @property
    def n_seqs(self) -> int:
        return len(self.seq_lens)

    @property
    def total_tokens(self) -> int:
        return int(sum(self.seq_lens))


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def place_spans(n: int, k: int, lo: int, hi: int, rng: np.random.Generator
                ) -> List[Tuple[int, int]]:
    """k spans with lengths uniform on {lo..hi}, placed in [0, n).

    Gaps come from k sorted uniform cut points of the free length, so spans
    keep their order and may touch.  Lengths are redrawn while they do not fit.
    """
    for _ in range(10000):
        lens = rng.integers(lo, hi + 1, size=k)
        free = n - int(lens.sum())
        if free >= 0:
            break
    else:
        raise ValueError("place_spans: spans never fit")
    cuts = np.sort(rng.integers(0, free + 1, size=k))
    gaps = np.diff(np.concatenate([[0], cuts, [free]]))
    out, o = [], int(gaps[0])
    for j in range(k):
        out.append((o, int(lens[j])))
        o += int(lens[j]) + int(gaps[j + 1])
    return out


def spans_to_mask(n: int, spans: List[Tuple[int, int]]) -> np.ndarray:
    m = np.zeros(n, dtype=np.uint8)
    for s, l in spans:
        m[s:s + l] = 1
    return m


# ---------------------------------------------------------------------------
# The workloads (named by what they are)
# ---------------------------------------------------------------------------
SHAPES: Dict[str, Shape] = {
    "one_layer_4k": Shape(1, 8, 128, 32, 1.0e4),
    "llama8b_32k": Shape(32, 8, 128, 32, 5.0e5),
    "ragged_batch_64": Shape(32, 8, 128, 32, 5.0e5),
    "history_50_turns": Shape(36, 8, 64, 64, 1.5e5),
    "llama70b_4x64k": Shape(80, 8, 128, 64, 5.0e5),
}


def one_layer_4k() -> Workload:
    """1 layer, 8 kv heads, d=128, 4096 tokens; drop [1024, 2048); 32 q heads."""
    n = 4096
    sp = [(1024, 1024)]
    return Workload("one_layer_4k", SHAPES["one_layer_4k"], [n], [spans_to_mask(n, sp)], None, 101,
                    "single sequence, 1 layer, span [1024,2048) dropped", [sp])


def llama8b_32k() -> Workload:
    """Llama-3.1-8B shape, 32768 tokens, six tool spans of 1024..4096 tokens."""
    rng = _rng(2)
    n = 32768
    sp = place_spans(n, 6, 1024, 4096, rng)
    return Workload("llama8b_32k", SHAPES["llama8b_32k"], [n], [spans_to_mask(n, sp)], None, 102,
                    "Llama-8B shape, 32768 tokens, 6 tool spans dropped", [sp])


def _span_batch(name: str, lens: np.ndarray, frac: float, rng, shuffle: bool,
                data_seed: int, desc: str) -> Workload:
    masks, spans = [], []
    for n in lens:
        k = max(1, int(round(frac * int(n) / 2560)))
        sp = place_spans(int(n), k, 1024, 4096, rng)
        spans.append(sp)
        masks.append(spans_to_mask(int(n), sp))
    n_pages = int(sum((int(n) + BLOCK - 1) // BLOCK for n in lens))
    order = rng.permutation(n_pages).astype(np.int32) if shuffle else None
    return Workload(name, SHAPES[name], [int(n) for n in lens], masks, order,
                    data_seed, desc, spans)


def ragged_batch_64(n_seqs: int = 64) -> Workload:
    """64 ragged sequences, lengths lognormal (median 16K, sigma 0.5, clipped
    to [8K, 64K]), shuffled page table, tool spans covering ~40% of tokens."""
    rng = _rng(3)
    z = rng.standard_normal(64)
    lens = np.clip(np.round(16384 * np.exp(0.5 * z)), 8192, 65536).astype(np.int64)
    return _span_batch("ragged_batch_64", lens[:n_seqs], 0.4, rng, True, 103,
                       "64 ragged sequences, shuffled pages, ~40% dropped")


def llama70b_4x64k() -> Workload:
    """Llama-3.1-70B shape, 4 x 65536 tokens, tool spans covering ~50%."""
    rng = _rng(5)
    return _span_batch("llama70b_4x64k", np.full(4, 65536, dtype=np.int64), 0.5, rng, False,
                       105, "Llama-70B shape, 4 x 65536 tokens, ~50% dropped")


# ---------------------------------------------------------------------------
# Long operation history of an agent run
# ---------------------------------------------------------------------------
@dataclass
class History:
    """Message-level op list of a long agent run.

    ops items: ("append", msg_id, n_tokens) | ("drop", [msg_ids]) |
               ("repos",) | ("drop_repos", [msg_ids]).
    Message m owns the global token ids [msg_start[m], msg_start[m] + msg_len[m]).
    """
    msg_len: List[int]
    msg_start: List[int]
    ops: List[tuple]
    total_tokens: int

    def max_active(self) -> int:
        """Largest number of active tokens at any point of the run (message
        lengths only: appends add a message, drops remove listed ones)."""
        alive, n, top = set(), 0, 0
        for op in self.ops:
            if op[0] == "append":
                alive.add(op[1])
                n += op[2]
                top = max(top, n)
            elif op[0] in ("drop", "drop_repos"):
                for m in op[1]:
                    if m in alive:
                        alive.discard(m)
                        n -= self.msg_len[m]
        return top


def history_50_turns(seed: int = 4, turns: int = 50, total: int = 131072,
               keep_turns: int = 3, repos_every: int = 3,
               assistant_range: Tuple[int, int] = (64, 512),
               tool_range: Tuple[int, int] = (512, 8192)) -> History:
    """50 turns of (assistant 64..512 tokens, tool response 512..8192 tokens).

    Lengths lo + c*(hi-lo)*w with w ~ U(0,1) and one common c chosen so the
    run totals exactly `total` tokens (floors, remainder on the last tool
    response).  At the end of turn t >= keep_turns+1 the tool response of turn
    t-keep_turns is dropped; every `repos_every`-th turn repositions (fused
    after that turn's drop; the first one has nothing to drop).
    """
    rng = _rng(seed)
    a = rng.uniform(size=turns)
    u = rng.uniform(size=turns)
    (lo_a, hi_a), (lo_u, hi_u) = assistant_range, tool_range
    need = total - turns * (lo_a + lo_u)
    c = need / ((hi_a - lo_a) * a.sum() + (hi_u - lo_u) * u.sum())
    if not 0.0 < c <= 1.0:
        raise ValueError("history_50_turns: lengths cannot reach the total within range")
    A = np.floor(lo_a + c * (hi_a - lo_a) * a).astype(np.int64)
    U = np.floor(lo_u + c * (hi_u - lo_u) * u).astype(np.int64)
    U[-1] += total - int(A.sum() + U.sum())
    msg_len, msg_start, ops = [], [], []
    cur = 0
    for t in range(1, turns + 1):
        for n in (int(A[t - 1]), int(U[t - 1])):
            mid = len(msg_len)
            msg_len.append(n)
            msg_start.append(cur)
            cur += n
            ops.append(("append", mid, n))
        drop = [2 * (t - keep_turns - 1) + 1] if t > keep_turns else []
        rep = (t % repos_every == 0)
        if drop and rep:
            ops.append(("drop_repos", drop))
        elif drop:
            ops.append(("drop", drop))
        elif rep:
            ops.append(("repos",))
    return History(msg_len, msg_start, ops, cur)


def mask_for_messages(token_ids: np.ndarray, hist: History, msg_ids) -> np.ndarray:
    """u8 mask over the active entries (given by their token ids) that belong
    to the listed messages."""
    m = np.zeros(token_ids.shape[0], dtype=np.uint8)
    for mid in msg_ids:
        s = hist.msg_start[mid]
        m |= ((token_ids >= s) & (token_ids < s + hist.msg_len[mid])).astype(np.uint8)
    return m


WORKLOADS = {"one_layer_4k": one_layer_4k, "llama8b_32k": llama8b_32k,
             "ragged_batch_64": ragged_batch_64, "llama70b_4x64k": llama70b_4x64k}


@dataclass
class Restore:
    """A request re-run after eviction as segments ([CE] Appendix A.1.1).

    versions[j] = (drop mask over the source sequence, rows of segment j):
    version j is the source with that mask dropped and its survivors moved
    to canonical positions; its last `rows` entries are segment j's tokens.
    """
    name: str
    shape: Shape
    n_tokens: int
    versions: List[Tuple[np.ndarray, int]]
    data_seed: int
    description: str = ""


def restore_llama8b_32k() -> Restore:
    """The Llama-8B-shaped request (32768 tokens, six tool spans) recomputed in seven
    segments.  Segment 0 is the text before the first span; segment j >= 1
    is tool span j plus the text up to the next span.  Span j stays visible
    to its own segment and is dropped (with reposition) before the next one,
    so segment j attends over: the text of segments 0..j-1 without their
    spans, then its own tokens."""
    wl = llama8b_32k()
    n = wl.seq_lens[0]
    sp = sorted(wl.spans[0])
    starts = [0] + [s for s, _ in sp] + [n]
    versions = []
    for j in range(len(sp) + 1):
        lo, hi = starts[j], starts[j + 1]
        m = np.zeros(n, dtype=np.uint8)
        for s, ln in sp[:max(0, j - 1)]:
            m[s:s + ln] = 1
        m[hi:] = 1
        versions.append((m, hi - lo))
    return Restore("restore_llama8b_32k", wl.shape, n, versions, wl.data_seed,
                   "the Llama-8B-shaped request restored in 7 segments over 7 position versions")


# ---------------------------------------------------------------------------
# bf16 ~N(0,1) tensors
# ---------------------------------------------------------------------------
def randn_bf16(shape, seed: int, device: str = "cpu"):
    """bf16 tensor of N(0,1) draws from a torch generator seeded with `seed`."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return torch.randn(tuple(shape), generator=g, dtype=torch.float32,
                       device=device).to(torch.bfloat16)
