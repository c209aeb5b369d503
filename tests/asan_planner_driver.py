"""Drives the host planner (fa_plan.cpp) built with AddressSanitizer and UndefinedBehaviorSanitizer
through its host-only C entry points, over the argument ranges where its int64 clamping and
overflow guards work: sentinel pre/next values, empty and single-element batches, long varlen
lists, large sizes near the supported limits, paged-cache checks and mode-1 sizing.

Run by tests/test_planner_sanitized.py in a child process with the sanitizer runtime preloaded;
any finding aborts the process (exit status != 0). Prints "planner sanitized run ok" at the end.
"""

import ctypes
import random
import sys

lib = ctypes.CDLL(sys.argv[1])
i32, i64, f32, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t


class Dims(ctypes.Structure):
    _fields_ = [("dtype", i32), ("B", i64), ("N", i64), ("Sq", i64), ("Skv", i64), ("D", i64),
                ("T_q", i64), ("T_kv", i64)]


class Stats(ctypes.Structure):
    _fields_ = [("kernel", i32), ("block_m", i32), ("block_n", i32), ("work_items", i64),
                ("kv_tiles_visited", i64), ("kv_tiles_full", i64), ("kv_tiles_total", i64),
                ("workspace_bytes", sz), ("launch_order", i32), ("edge_skip", i32)]


class Paged(ctypes.Structure):
    _fields_ = [("block_table", ctypes.c_void_p), ("max_blocks_per_seq", i64), ("num_blocks", i64),
                ("block_size", i64), ("cache_layout", i32), ("reserved", i32)]


P64 = ctypes.POINTER(i64)
lib.fa_plan_stats_get.argtypes = [ctypes.POINTER(Dims), i32, i32, i64, i64, P64, P64, P64, i32, i32, f32,
                                  ctypes.POINTER(Stats)]
lib.fa_fwd_workspace_size.argtypes = [ctypes.POINTER(Dims), i32, i32, P64, P64, ctypes.POINTER(sz)]
lib.fa_fwd_mask_workspace_size.argtypes = [ctypes.POINTER(Dims), i32, P64, ctypes.POINTER(sz)]
lib.fa_fwd_paged_workspace_size.argtypes = [ctypes.POINTER(Dims), i32, i32, P64, P64, ctypes.POINTER(Paged),
                                            ctypes.POINTER(sz)]
lib.fa_tile_shape.argtypes = [ctypes.POINTER(Dims), i32, P64, P64, ctypes.POINTER(i32), ctypes.POINTER(i32), P64,
                              P64]
lib.fa_status_str.restype = ctypes.c_char_p


def arr(vals):
    if vals is None:
        return None
    return (i64 * max(len(vals), 1))(*vals)


def stats(d, layout, mode, pre=0, nxt=0, ql=None, kl=None, prefix=None, alibi=0, mask=0, scale=0.1):
    s = Stats()
    return lib.fa_plan_stats_get(ctypes.byref(d), layout, mode, pre, nxt, arr(ql), arr(kl), arr(prefix), alibi, mask,
                                 scale, ctypes.byref(s))


def cum(xs):
    out, t = [], 0
    for x in xs:
        t += x
        out.append(t)
    return out


BIG = 2 ** 63 - 1
rng = random.Random(7)
n_calls = 0
for code in range(-1, 8):
    assert lib.fa_status_str(code)
# Sentinels and extremes of pre/next in every mode, fixed-length layouts.
for mode in range(9):
    for pre, nxt in [(BIG, BIG), (-BIG - 1, BIG), (BIG, -BIG - 1), (0, 0), (2 ** 40, -2 ** 40), (-5, 2 ** 33),
                     (2 ** 31, 2 ** 31), (-(2 ** 31), 2 ** 31 - 1)]:
        for (B, N, Sq, Skv, D) in [(0, 1, 0, 0, 1), (1, 1, 1, 1, 128), (2, 3, 0, 7, 64), (2, 3, 7, 0, 64),
                                   (1, 1, 2 ** 27, 2 ** 27, 128), (3, 4, 300, 1, 16), (2 ** 14, 2, 3, 3, 8),
                                   (1, 2 ** 16, 16, 16, 128)]:
            for dtype in (0, 1, 2):
                for layout in (0, 1):
                    d = Dims(dtype, B, N, Sq, Skv, D, 0, 0)
                    prefix = [rng.randrange(0, 2 ** 40) for _ in range(min(B, 64))] if B <= 64 else None
                    stats(d, layout, mode, pre, nxt, prefix=prefix, alibi=mode % 2, mask=1)
                    n_calls += 1
                    out = sz(0)
                    lib.fa_fwd_workspace_size(ctypes.byref(d), layout, mode, None, None, ctypes.byref(out))
                    if mode == 1:
                        for bc in ([0, 0], [1, 0], [0, 1], [1, 1]):
                            lib.fa_fwd_mask_workspace_size(ctypes.byref(d), layout, arr(bc), ctypes.byref(out))
# Varlen TND: empty sequences, one long list, non-monotone and inconsistent totals, modes 7 / 8 edges.
for trial in range(60):
    nb = rng.choice([0, 1, 2, 5, 17, 1000])
    ql = [rng.choice([0, 0, 1, 5, 128, 257, 4096, 2 ** 20]) for _ in range(nb)]
    kl = [rng.choice([0, 1, 7, 128, 300, 5000, 2 ** 21]) for _ in range(nb)]
    if trial % 5 == 4 and nb > 1:
        ql[0] = -3
    cq, ck = cum(ql), cum(kl)
    if trial % 7 == 6 and nb > 1:
        cq[1], cq[0] = cq[0], cq[1] + 1
    d = Dims(2, nb, 4, 0, 0, 128, cq[-1] if cq else 0, ck[-1] if ck else 0)
    for mode in (0, 2, 3, 5, 7, 8):
        pre = rng.choice([0, BIG, -BIG - 1, 2 ** 30, max(kl + [0])])
        nxt = rng.choice([0, BIG, -BIG - 1, -(2 ** 30), -max(ql + [0])])
        stats(d, 2, mode, pre, nxt, cq, ck, prefix=[rng.randrange(0, 10 ** 6) for _ in range(nb)])
        n_calls += 1
    out = sz(0)
    lib.fa_fwd_workspace_size(ctypes.byref(d), 2, 3, arr(cq), arr(ck), ctypes.byref(out))
    bm, bn, nq, nk = i32(0), i32(0), i64(0), i64(0)
    lib.fa_tile_shape(ctypes.byref(d), 2, arr(cq), arr(ck), ctypes.byref(bm), ctypes.byref(bn), ctypes.byref(nq),
                      ctypes.byref(nk))
# Short-query (split-KV decode) planning, fixed and varlen.
for Skv in (0, 1, 63, 64, 4097, 2 ** 20, 2 ** 27):
    for B, N in ((1, 1), (4, 32), (64, 64), (2 ** 12, 8)):
        stats(Dims(2, B, N, 1, Skv, 128, 0, 0), 0, 3)
        n_calls += 1
# Paged caches: sizes around the limits.
for bs in (1, 16, 64, 128, 2 ** 24, 2 ** 24 + 1):
    for nb in (1, 7, 2 ** 31 - 1, 2 ** 31):
        for mbps in (1, 3, 2 ** 24, 2 ** 24 + 1):
            for layout_c in (0, 1, 2):
                pk = Paged(None, mbps, nb, bs, layout_c, 0)
                out = sz(0)
                lib.fa_fwd_paged_workspace_size(ctypes.byref(Dims(2, 2, 8, 4, 5000, 128, 0, 0)), 0, 3, None, None,
                                                ctypes.byref(pk), ctypes.byref(out))
                n_calls += 1
# A few statuses the rules fix, so the run also checks that validation still answers.
d = Dims(2, 2, 4, 300, 500, 128, 0, 0)
assert stats(d, 0, 4, BIG, BIG) == 0
assert stats(d, 0, 4, -(2 ** 40), 2 ** 40 - 1) == 2      # band with pre + next < 0
assert stats(d, 0, 4, -BIG - 1, BIG) == 2                 # below the accepted range
assert stats(d, 0, 4, 2 ** 62, 2 ** 62) == 0              # sum beyond int64 is still a valid band
assert stats(Dims(2, 0, 4, 300, 500, 128, 0, 0), 0, 3) == 0
assert stats(Dims(2, 1, 4, 2 ** 28, 8, 128, 0, 0), 0, 3) == 3
assert stats(Dims(2, 1, 4, 8, 8, 256, 0, 0), 0, 3) == 3
assert stats(Dims(2, 2, 4, 0, 0, 128, 9, 9), 2, 3, ql=[5, 4], kl=[5, 9]) == 2   # ends must grow
assert stats(Dims(2, 2, 4, 0, 0, 128, 9, 9), 2, 3, ql=[4, 9], kl=[5, 9]) == 0
print(f"planner sanitized run ok ({n_calls} planning calls)")
