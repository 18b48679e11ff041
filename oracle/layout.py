"""Memory order of the paged pool (TEST INFRASTRUCTURE).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU baseline may
import this module.
"""
from __future__ import annotations

import numpy as np


def kv_cache_stride_order(layout: str = "NHD"):
    """Order in which the pool's logical dimensions (blocks, K/V, slot, KV head,
    head size) are laid out in memory, outermost first.

    «FlashAttention y FlashInfer», §Motivación de diseño (two layouts NHD / HND,
    ``get_kv_cache_stride_order``): NHD keeps the logical order (a slot's heads
    are adjacent); HND puts the KV head before the slot, so one head's rows of a
    block are adjacent.  Reading: HND = physical (blocks, K/V, KV head, slot,
    head size).
    """
    if layout == "NHD":
        return (0, 1, 2, 3, 4)
    if layout == "HND":
        return (0, 1, 3, 2, 4)
    raise ValueError(f"layout {layout!r}")


def logical_pool(kv_cache: np.ndarray, layout: str = "NHD") -> np.ndarray:
    """The pool as (blocks, K/V, slot, KV head, head size) whatever its memory
    order: the physical array is indexed by the dimensions in stride order."""
    order = kv_cache_stride_order(layout)
    return np.transpose(kv_cache, np.argsort(order))
