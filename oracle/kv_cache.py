"""Paged KV cache: plain CPU definitions of the scatter and of reading K/V back by block table.

TEST INFRASTRUCTURE (see the package docstring): only the test suite and the benchmark's
CPU-baseline leg use it.

Source: "aclnnScatterPaKvCache" (ops-transformer doc), sections "功能说明" (scenarios two,
six and seven) and "约束说明". The operation updates the key and value caches at given
positions: token t of key [num_tokens, N, head_size] goes to the cache slot
slot_mapping[t], where slot = block * block_size + offset, for every head. Two cache
layouts:
- "Norm" (scenario two): cache [num_blocks, block_size, N, head_size];
- "NHSD" (scenario seven): cache [num_blocks, N, block_size, head_size].
Scenario six passes no value (keys only). Slots lie in [0, num_blocks * block_size - 1] and
do not repeat.

Reading: a slot outside that range (the page leaves it undefined; serving code marks padding
tokens with -1) writes nothing.
"""

from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

CACHE_LAYOUTS = ("Norm", "NHSD")


def _cache_index(layout: str, block: int, offset: int, h: int):
    if layout == "Norm":
        return (block, offset, h)
    if layout == "NHSD":
        return (block, h, offset)
    raise ValueError(layout)


def scatter_kv_cache(key: np.ndarray, key_cache: np.ndarray, slot_mapping: Sequence[int],
                     value: Optional[np.ndarray] = None, value_cache: Optional[np.ndarray] = None,
                     layout: str = "Norm"):
    """Returns copies of (key_cache, value_cache) with the tokens written, one (token, head)
    at a time: cache[slot // block_size, slot % block_size, h] = key[t, h] ("Norm")."""
    key = np.asarray(key)
    kc = np.array(key_cache, copy=True)
    vc = None if value_cache is None else np.array(value_cache, copy=True)
    block_size = kc.shape[1] if layout == "Norm" else kc.shape[2]
    n_slots = kc.shape[0] * block_size
    for t, slot in enumerate(slot_mapping):
        slot = int(slot)
        if slot < 0 or slot >= n_slots:
            continue
        block, offset = divmod(slot, block_size)
        for h in range(key.shape[1]):
            kc[_cache_index(layout, block, offset, h)] = key[t, h]
            if vc is not None:
                vc[_cache_index(layout, block, offset, h)] = value[t, h]
    return kc, vc


def gather_paged(cache: np.ndarray, block_table: Sequence[int], length: int,
                 layout: str = "Norm") -> np.ndarray:
    """Rows 0 .. length-1 of one sequence whose pages are block_table (in order), as an
    array [length, N, head_size]: row j lives in page block_table[j // block_size] at offset
    j % block_size."""
    block_size = cache.shape[1] if layout == "Norm" else cache.shape[2]
    n = cache.shape[2] if layout == "Norm" else cache.shape[1]
    out = np.zeros((length, n, cache.shape[3]), dtype=cache.dtype)
    for j in range(length):
        page, offset = block_table[j // block_size], j % block_size
        for h in range(n):
            out[j, h] = cache[_cache_index(layout, page, offset, h)]
    return out
