"""Pins for the paged-KV-cache oracle (CPU only): "aclnnScatterPaKvCache", sections 功能说明
(scenarios two, six and seven) and 约束说明."""

import json
import os

import numpy as np

from oracle import kv_cache

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _key(t, n, d):
    return (100 * np.arange(t)[:, None, None] + 10 * np.arange(n)[None, :, None]
            + np.arange(d)[None, None, :]).astype(np.float64)


def test_golden_scatter_example():
    """The hand-derived tiny example (golden file): slot s lands in block s // block_size at
    offset s % block_size, for every head; nothing else changes."""
    g = json.load(open(os.path.join(GOLDEN, "kv_scatter_example.json")))
    nb, bs, n, d = g["num_blocks"], g["block_size"], g["num_head"], g["head_size"]
    key = _key(len(g["slot_mapping"]), n, d)
    kc, vc = kv_cache.scatter_kv_cache(key, np.full((nb, bs, n, d), -1.0), g["slot_mapping"])
    assert vc is None
    assert kc.tolist() == g["expected_norm_cache"]


def test_scatter_then_read_by_slot_returns_tokens():
    """Reading the Norm cache flattened to [num_blocks * block_size, N, D] at the slots gives
    the tokens back (numpy reshape, not the oracle's loop); other slots keep their values."""
    rng = np.random.default_rng(5)
    nb, bs, n, d, t = 7, 4, 3, 8, 11
    slots = rng.permutation(nb * bs)[:t]
    key, val = rng.standard_normal((t, n, d)), rng.standard_normal((t, n, d))
    k0, v0 = rng.standard_normal((nb, bs, n, d)), rng.standard_normal((nb, bs, n, d))
    kc, vc = kv_cache.scatter_kv_cache(key, k0, slots, val, v0)
    flat_k, flat_v = kc.reshape(nb * bs, n, d), vc.reshape(nb * bs, n, d)
    np.testing.assert_array_equal(flat_k[slots], key)
    np.testing.assert_array_equal(flat_v[slots], val)
    rest = np.setdiff1d(np.arange(nb * bs), slots)
    np.testing.assert_array_equal(flat_k[rest], k0.reshape(nb * bs, n, d)[rest])
    np.testing.assert_array_equal(flat_v[rest], v0.reshape(nb * bs, n, d)[rest])


def test_nhsd_is_norm_with_heads_before_rows():
    """Scenario seven's cache [num_blocks, N, block_size, D] holds the same data as the Norm
    cache with axes 1 and 2 swapped."""
    rng = np.random.default_rng(6)
    nb, bs, n, d, t = 5, 8, 4, 16, 20
    slots = rng.permutation(nb * bs)[:t]
    key = rng.standard_normal((t, n, d))
    k0 = rng.standard_normal((nb, bs, n, d))
    norm, _ = kv_cache.scatter_kv_cache(key, k0, slots)
    nhsd, _ = kv_cache.scatter_kv_cache(key, k0.transpose(0, 2, 1, 3).copy(), slots, layout="NHSD")
    np.testing.assert_array_equal(nhsd, norm.transpose(0, 2, 1, 3))


def test_out_of_range_slots_write_nothing():
    """Slots outside [0, num_blocks * block_size - 1] (e.g. -1 for padding) change nothing."""
    rng = np.random.default_rng(7)
    nb, bs, n, d = 3, 4, 2, 4
    key = rng.standard_normal((3, n, d))
    k0 = rng.standard_normal((nb, bs, n, d))
    kc, _ = kv_cache.scatter_kv_cache(key, k0, [-1, nb * bs, 2 ** 40])
    np.testing.assert_array_equal(kc, k0)


def test_gather_by_block_table_inverts_scatter():
    """Tokens 0..L-1 of a sequence scattered to slots table[j // bs] * bs + j % bs are read
    back in order by the block table."""
    rng = np.random.default_rng(8)
    nb, bs, n, d, L = 9, 4, 2, 8, 13
    table = list(rng.permutation(nb)[:4])
    slots = [table[j // bs] * bs + j % bs for j in range(L)]
    key = rng.standard_normal((L, n, d))
    for layout in kv_cache.CACHE_LAYOUTS:
        shape = (nb, bs, n, d) if layout == "Norm" else (nb, n, bs, d)
        kc, _ = kv_cache.scatter_kv_cache(key, np.zeros(shape), slots, layout=layout)
        np.testing.assert_array_equal(kv_cache.gather_paged(kc, table, L, layout), key)
