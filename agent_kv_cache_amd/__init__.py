"""MI355X-native hot path of agent cache engineering.

drop (order-preserving compaction of a paged bf16 KV cache), reposition
(RoPE re-rotation of surviving keys to new positions) and decode attention
over the active KV, as HIP kernels for gfx950 behind the C ABI of
include/akv.h.  `binding` marshals arguments to libakv.so; `workloads` and
`harness` make seeded synthetic inputs.
"""
from .binding import AkvCache, AkvError, lib  # noqa: F401

__all__ = ["AkvCache", "AkvError", "lib"]
