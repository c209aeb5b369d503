"""C-ABI boundary tests that need no GPU: the library loads, exports every declared entry
point, validates arguments with the documented status codes before any device work, and
its host-side tile planning agrees with brute force over the oracle's mask."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from masked_attention_forward_amd import binding as fb
from masked_attention_forward_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, NULLPTR, INVALID, UNSUPPORTED, HIPERR, WORKSPACE = 0, 1, 2, 3, 4, 5


@pytest.fixture(scope="module")
def lib():
    return fb.load_library()


def declared_functions():
    names = []
    for hdr in os.listdir(os.path.join(ROOT, "include")):
        if not hdr.endswith(".h"):
            continue
        text = open(os.path.join(ROOT, "include", hdr)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(fa_[a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"fa_fwd", "fa_fwd_workspace_size", "fa_mask_probe", "fa_status_str"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_exp2_rate_probe_argument_checks(lib):
    # Rejected before any device call, so these run without a GPU.
    n = ctypes.c_int64(0)
    assert lib.fa_exp2_rate_probe(None, 1, 1, ctypes.byref(n), None) == 1
    fake = ctypes.c_void_p(256)
    assert lib.fa_exp2_rate_probe(fake, 1, 1, None, None) == 1
    for blocks, iters in ((0, 1), (1, 0), (-1, 5), (1 << 21, 1), (1, 1 << 21)):
        assert lib.fa_exp2_rate_probe(fake, blocks, iters, ctypes.byref(n), None) == 2


def test_status_strings(lib):
    for code in range(6):
        assert fb.fa_status_str(code).startswith(fb.STATUS_NAMES[code])


def _stats_status(lib, dims, layout, mode, pre=0, nxt=0, qlen=None, kvlen=None, prefix=None,
                  alibi=False, mask=False, scale=0.125):
    s = fb.FaPlanStats()
    return lib.fa_plan_stats_get(ctypes.byref(dims) if dims is not None else None, layout, mode, pre, nxt,
                                 fb._i64(qlen), fb._i64(kvlen), fb._i64(prefix), int(alibi), int(mask),
                                 scale, ctypes.byref(s))


def bnsd(B=2, N=4, Sq=64, Skv=64, D=128, dtype=2):
    return fb.make_dims(dtype, 0, B=B, N=N, Sq=Sq, Skv=Skv, D=D)


def tnd(qlens, kvlens, N=2, D=128, dtype=2):
    return fb.make_dims(dtype, 2, B=len(qlens), N=N, D=D, T_q=sum(qlens), T_kv=sum(kvlens))


def test_generic_validation(lib):
    assert _stats_status(lib, None, 0, 3) == NULLPTR
    assert _stats_status(lib, bnsd(dtype=7), 0, 3) == INVALID
    assert _stats_status(lib, bnsd(), 5, 3) == INVALID
    assert _stats_status(lib, bnsd(), 0, 9) == INVALID
    assert _stats_status(lib, bnsd(), 0, -1) == INVALID
    assert _stats_status(lib, bnsd(N=0), 0, 3) == INVALID
    assert _stats_status(lib, bnsd(Sq=-1), 0, 3) == INVALID
    assert _stats_status(lib, bnsd(D=256), 0, 3) == UNSUPPORTED
    assert _stats_status(lib, bnsd(), 0, 3, scale=0.0) == INVALID
    assert _stats_status(lib, bnsd(), 0, 3, scale=-0.1) == INVALID
    assert _stats_status(lib, bnsd(), 0, 3, scale=float("nan")) == INVALID
    assert _stats_status(lib, bnsd(), 0, 3) == OK
    assert _stats_status(lib, bnsd(B=0), 0, 3) == OK
    assert _stats_status(lib, bnsd(Sq=0, Skv=0), 0, 3) == OK


def test_alibi_rules(lib):
    # "压缩mask", constraints: alibi needs head size <= 128.
    assert _stats_status(lib, bnsd(D=192), 0, 3, alibi=True) == INVALID
    assert _stats_status(lib, bnsd(D=128), 0, 3, alibi=True) == OK
    # "sparseMode介绍", sparseMode=7/8: the optional pse input is not supported.
    q, k = [3, 2], [3, 6]
    assert _stats_status(lib, tnd(q, k), 2, 7, 6, -2, synth.cumulative_ends(q), synth.cumulative_ends(k),
                         alibi=True) == INVALID


def test_mode0_band_sign_rules(lib):
    """sparseMode=0: negative next needs pre >= |next| and |next| < Skv; negative pre needs
    next >= |pre| and |pre| < Sq."""
    d = bnsd(Sq=16, Skv=16)
    assert _stats_status(lib, d, 0, 0, 9, -3) == OK
    assert _stats_status(lib, d, 0, 0, 2, -3) == INVALID
    assert _stats_status(lib, d, 0, 0, 20, -16) == INVALID
    assert _stats_status(lib, d, 0, 0, -3, 7) == OK
    assert _stats_status(lib, d, 0, 0, -3, 2) == INVALID
    assert _stats_status(lib, d, 0, 0, -16, 20) == INVALID
    assert _stats_status(lib, d, 0, 0, 2**63 - 1, 2**63 - 1) == OK
    assert _stats_status(lib, d, 0, 0, -2**63, 5) == INVALID


def test_mode4_must_intersect(lib):
    d = bnsd(Sq=16, Skv=24)
    assert _stats_status(lib, d, 0, 4, 3, -3) == OK
    assert _stats_status(lib, d, 0, 4, 3, -4) == INVALID
    assert _stats_status(lib, d, 0, 4, 1024, 0) == OK


def test_mode7_mode8_rules_from_page_examples(lib):
    """The worked examples of sparseMode=7 / 8 pass; moving pre or next past the stated
    limits fails; both modes need the TND layout."""
    q7, k7 = [3, 2], [3, 6]
    cq, ck = synth.cumulative_ends(q7), synth.cumulative_ends(k7)
    d7 = tnd(q7, k7)
    assert _stats_status(lib, d7, 2, 7, 6, -2, cq, ck) == OK
    assert _stats_status(lib, d7, 2, 7, 5, -2, cq, ck) == INVALID      # pre < last Skv
    assert _stats_status(lib, d7, 2, 7, 6, 1, cq, ck) == INVALID       # next > 0
    assert _stats_status(lib, d7, 2, 7, 6, -5, cq, ck) == INVALID      # next < last_Sq - last_Skv
    assert _stats_status(lib, d7, 2, 7, 6, -4, cq, ck) == OK
    # a non-band batch with Sq > Skv
    qb, kb = [4, 2], [3, 6]
    assert _stats_status(lib, tnd(qb, kb), 2, 7, 6, -2, synth.cumulative_ends(qb),
                         synth.cumulative_ends(kb)) == INVALID
    q8, k8 = [3, 5, 4], [4, 5, 4]
    cq, ck = synth.cumulative_ends(q8), synth.cumulative_ends(k8)
    d8 = tnd(q8, k8)
    assert _stats_status(lib, d8, 2, 8, 4, 1, cq, ck) == OK
    assert _stats_status(lib, d8, 2, 8, 3, 1, cq, ck) == INVALID       # pre < first Skv
    assert _stats_status(lib, d8, 2, 8, 4, -2, cq, ck) == INVALID      # next < first_Sq - first_Skv
    assert _stats_status(lib, d8, 2, 8, 4, -1, cq, ck) == OK
    assert _stats_status(lib, bnsd(), 0, 7, 64, 0) == INVALID
    assert _stats_status(lib, bnsd(), 1, 8, 64, 0) == INVALID


def test_varlen_array_rules(lib):
    d = tnd([3, 2], [3, 6])
    assert _stats_status(lib, d, 2, 3, qlen=None, kvlen=[3, 9]) == NULLPTR
    assert _stats_status(lib, d, 2, 3, qlen=[3, 5], kvlen=[3, 9]) == OK
    assert _stats_status(lib, d, 2, 3, qlen=[3, 2], kvlen=[3, 9]) == INVALID   # not cumulative
    assert _stats_status(lib, d, 2, 3, qlen=[3, 6], kvlen=[3, 9]) == INVALID   # T_q mismatch
    assert _stats_status(lib, d, 2, 3, qlen=[-1, 5], kvlen=[3, 9]) == INVALID


def test_prefix_and_mask_rules(lib):
    d = bnsd()
    assert _stats_status(lib, d, 0, 5) == NULLPTR
    assert _stats_status(lib, d, 0, 5, prefix=[3, 9]) == OK
    assert _stats_status(lib, d, 0, 6, prefix=[3, -1]) == INVALID
    assert _stats_status(lib, d, 0, 1) == NULLPTR
    assert _stats_status(lib, d, 0, 1, mask=True) == OK
    assert _stats_status(lib, tnd([3], [3]), 2, 1, qlen=[3], kvlen=[3], mask=True) == UNSUPPORTED


def test_fwd_rejects_before_device_work(lib):
    """fa_fwd returns its status before touching the GPU: null data pointers, a too-small
    workspace and invalid arguments come back without a HIP call (this host has no GPU)."""
    buf = (ctypes.c_char * 4096)()
    p = ctypes.cast(buf, ctypes.c_void_p)
    d = bnsd()
    right, sqrt_, left = 0, 1, 2
    st = lib.fa_fwd(None, p, p, p, p, ctypes.byref(d), 0, 3, 0, 0, None, None, None, None, right, None,
                    None, 0.125, None, 0, None)
    assert st == NULLPTR
    d2 = tnd([3, 2], [3, 6])
    need = fb.fa_fwd_workspace_size(d2, "TND", 3, [3, 5], [3, 9])
    assert need > 0
    st = lib.fa_fwd(p, p, p, p, p, ctypes.byref(d2), 2, 3, 0, 0, fb._i64([3, 5]), fb._i64([3, 9]), None,
                    None, right, None, None, 0.125, p, need - 1, None)
    assert st == WORKSPACE
    st = lib.fa_fwd(p, p, p, p, p, ctypes.byref(d2), 2, 3, 0, 0, fb._i64([3, 5]), fb._i64([3, 9]), None,
                    None, right, None, None, 0.125, None, 0, None)
    assert st == NULLPTR
    st = lib.fa_fwd(p, p, p, p, p, ctypes.byref(d), 0, 4, 3, -9, None, None, None, None, right, None,
                    None, 0.125, None, 0, None)
    assert st == INVALID
    # alibi_mode outside FA_ALIBI_RIGHT / FA_ALIBI_SQRT / FA_ALIBI_LEFT is rejected, with or
    # without slopes
    for bad in (-1, 3, 99):
        for slopes in (None, p):
            st = lib.fa_fwd(p, p, p, p, p, ctypes.byref(d), 0, 3, 0, 0, None, None, None, slopes, bad,
                            None, None, 0.125, None, 0, None)
            assert st == INVALID, (bad, slopes)
    # alibi (any variant) is not allowed with the split modes 7/8
    for mode in (right, sqrt_, left):
        st = lib.fa_fwd(p, p, p, p, p, ctypes.byref(d2), 2, 7, 3, 0, fb._i64([3, 5]), fb._i64([3, 9]), None,
                        p, mode, None, None, 0.125, p, need, None)
        assert st == INVALID, mode
    # empty problem: nothing to do, OK without pointers
    d0 = bnsd(B=0)
    st = lib.fa_fwd(None, None, None, None, None, ctypes.byref(d0), 0, 3, 0, 0, None, None, None, None,
                    right, None, None, 0.125, None, 0, None)
    assert st == OK


def test_workspace_size(lib):
    assert fb.fa_fwd_workspace_size(bnsd(), "BNSD", 3) == 0
    assert fb.fa_fwd_workspace_size(bnsd(), "BNSD", 5) > 0
    d = tnd([300, 7], [300, 9])
    n = fb.fa_fwd_workspace_size(d, "TND", 3, [300, 307], [300, 309])
    bm, bn, nq, nk = fb.fa_tile_shape(d, "TND", [300, 307], [300, 309])
    assert (bm, bn) == (256, 64)
    assert nq == 2 + 1 and nk == 5
    assert n >= 2 * 32 + nq * 8
    d32 = tnd([300, 7], [300, 9], dtype=0, D=16)
    bm, bn, nq, nk = fb.fa_tile_shape(d32, "TND", [300, 307], [300, 309])
    assert (bm, bn) == (64, 16)


# ---------------------------------------------------------------------------------------
# Host tile planning vs brute force over the oracle's mask
# ---------------------------------------------------------------------------------------

def brute_tiles(vis, bm, bn):
    """(visited, full) tile counts for one batch from an explicit visible matrix: a tile is
    visited iff it holds a visible entry; full iff it lies inside the sequence and every
    entry of its in-range rows is visible."""
    sq, skv = vis.shape
    visited = full = 0
    for i0 in range(0, sq, bm):
        for j0 in range(0, skv, bn):
            blk = vis[i0:i0 + bm, j0:j0 + bn]
            if blk.any():
                visited += 1
                if j0 + bn <= skv and blk.all():
                    full += 1
    return visited, full


def _random_case(rng, mode):
    sq = int(rng.integers(0, 300))
    skv = int(rng.integers(0, 300))
    if mode in (7,):
        skv = max(skv, sq)
    while True:
        pre = int(rng.integers(-sq, sq + skv + 3))
        nxt = int(rng.integers(-skv, sq + skv + 3))
        if mode == 0:
            if nxt < 0 and not (pre >= -nxt and -nxt < max(skv, 1)):
                continue
            if pre < 0 and not (nxt >= -pre and -pre < max(sq, 1)):
                continue
        if mode == 4 and pre + nxt < 0:
            continue
        return sq, skv, pre, nxt


@pytest.mark.parametrize("mode", [0, 2, 3, 4, 5, 6])
@pytest.mark.parametrize("dtype,D", [(2, 128), (0, 16)])
def test_plan_tiles_match_brute_force(lib, mode, dtype, D):
    rng = np.random.default_rng(500 + mode + 17 * dtype)
    for _ in range(12):
        sq, skv, pre, nxt = _random_case(rng, mode)
        B = 2
        prefix = [int(rng.integers(0, skv + 3)) for _ in range(B)]
        d = bnsd(B=B, N=1, Sq=sq, Skv=skv, D=D, dtype=dtype)
        st = fb.fa_plan_stats(d, "BNSD", mode, pre_tokens=pre, next_tokens=nxt, prefix=prefix, scale=0.1)
        bm, bn = st["block_m"], st["block_n"]
        vis_tot = full_tot = total = 0
        for b in range(B):
            vis = oracle.visible_matrix(mode, sq, skv, pre_tokens=pre, next_tokens=nxt, prefix_len=prefix[b])
            v, f = brute_tiles(vis, bm, bn)
            vis_tot += v
            full_tot += f
            total += -(-sq // bm) * -(-skv // bn)
        assert st["kv_tiles_visited"] == vis_tot, (mode, sq, skv, pre, nxt, prefix)
        assert st["kv_tiles_full"] == full_tot, (mode, sq, skv, pre, nxt, prefix)
        assert st["kv_tiles_total"] == total


@pytest.mark.parametrize("mode", [3, 7, 8])
def test_plan_tiles_varlen_match_brute_force(lib, mode):
    rng = np.random.default_rng(600 + mode)
    for _ in range(10):
        nb = int(rng.integers(1, 5))
        ql = [int(x) for x in rng.integers(0, 260, nb)]
        kl = [int(x) for x in rng.integers(0, 260, nb)]
        if mode == 7:
            kl = [max(a, b) for a, b in zip(ql, kl)]
        band = oracle.band_batch_index(mode, ql, kl)
        pre = nxt = 0
        if band is not None:
            sqb, skb = ql[band], kl[band]
            pre = skb + int(rng.integers(0, 5))
            if mode == 7:
                nxt = int(rng.integers(sqb - skb, 1))
            else:
                nxt = sqb - skb + int(rng.integers(0, 5))
        d = tnd(ql, kl, N=1)
        cq, ck = synth.cumulative_ends(ql), synth.cumulative_ends(kl)
        st = fb.fa_plan_stats(d, "TND", mode, pre_tokens=pre, next_tokens=nxt, actual_seq_qlen=cq,
                              actual_seq_kvlen=ck, scale=0.1)
        vt = ft = 0
        for b in range(nb):
            vis = oracle.visible_matrix(mode, ql[b], kl[b], pre_tokens=pre, next_tokens=nxt, band=(b == band))
            v, f = brute_tiles(vis, st["block_m"], st["block_n"])
            vt += v
            ft += f
        assert (st["kv_tiles_visited"], st["kv_tiles_full"]) == (vt, ft), (ql, kl, pre, nxt)


# ---------------------------------------------------------------------------------------
# Paged KV cache scatter: host validation (no device work)
# ---------------------------------------------------------------------------------------

def test_scatter_kv_cache_validation(lib):
    """fa_scatter_kv_cache checks its arguments before any launch ("aclnnScatterPaKvCache",
    return-code table): missing pointers, unknown layout / element size / slot type, and
    non-positive sizes; an empty token list is a no-op."""
    buf = (ctypes.c_char * 4096)()
    p = ctypes.cast(buf, ctypes.c_void_p)

    def dims(**kw):
        base = dict(num_tokens=4, num_heads=2, k_head_size=8, v_head_size=8, num_blocks=3, block_size=2,
                    elem_bytes=2, slot_bytes=4)
        base.update(kw)
        return fb.FaKvCacheDims(**base)

    call = lambda d, key=p, val=p, kc=p, vc=p, slots=p, layout=0: lib.fa_scatter_kv_cache(
        key, val, kc, vc, slots, ctypes.byref(d) if d is not None else None, layout, None)
    assert call(None) == NULLPTR
    assert call(dims(), key=None) == NULLPTR
    assert call(dims(), kc=None) == NULLPTR
    assert call(dims(), slots=None) == NULLPTR
    assert call(dims(), val=None) == NULLPTR            # value_cache without value
    assert call(dims(), layout=2) == INVALID
    assert call(dims(elem_bytes=3)) == INVALID
    assert call(dims(slot_bytes=2)) == INVALID
    assert call(dims(num_heads=0)) == INVALID
    assert call(dims(block_size=0)) == INVALID
    assert call(dims(num_tokens=-1)) == INVALID
    assert call(dims(num_tokens=0), key=None, val=None, kc=None, vc=None, slots=None) == OK
    assert call(dims(num_heads=1 << 17)) == UNSUPPORTED


# ---------------------------------------------------------------------------------------
# Paged forward: host validation of the block-table description (no device work)
# ---------------------------------------------------------------------------------------

def test_fwd_paged_validation(lib):
    """fa_fwd_paged checks its fa_paged_kv before any launch: layout, reserved field, sizes,
    a block table long enough for the longest sequence, and the pointers it needs."""
    buf = (ctypes.c_char * 4096)()
    p = ctypes.cast(buf, ctypes.c_void_p)
    d = bnsd(B=2, N=4, Sq=64, Skv=300, D=128)

    def pk(**kw):
        base = dict(block_table=p.value, max_blocks_per_seq=3, num_blocks=8, block_size=128, cache_layout=0,
                    reserved=0)
        base.update(kw)
        return fb.FaPagedKv(**base)

    def call(paged, dims=d, mode=3, kc=p, vc=p):
        return lib.fa_fwd_paged(p, kc, vc, p, p, ctypes.byref(dims), 0, mode, 0, 0, None, None, None, None, 0,
                                None, None, ctypes.byref(paged) if paged is not None else None, 0.125, None, 0,
                                None)

    assert call(None) == NULLPTR
    assert call(pk(cache_layout=2)) == INVALID
    assert call(pk(cache_layout=-1)) == INVALID
    assert call(pk(reserved=1)) == INVALID
    assert call(pk(block_size=0)) == INVALID
    assert call(pk(num_blocks=0)) == INVALID
    assert call(pk(max_blocks_per_seq=0)) == INVALID
    assert call(pk(max_blocks_per_seq=2)) == INVALID        # 2 pages x 128 keys < 300 keys
    assert call(pk(block_size=64, max_blocks_per_seq=4)) == INVALID
    assert call(pk(num_blocks=1 << 32)) == UNSUPPORTED
    assert call(pk(block_table=None)) == NULLPTR
    assert call(pk(), kc=None) == NULLPTR
    assert call(pk(), vc=None) == NULLPTR
    assert call(pk(), mode=9) == INVALID                    # fa_fwd's own rules still hold
    # no keys anywhere: nothing is read, so no table is needed
    d0 = bnsd(B=2, N=4, Sq=64, Skv=0, D=128)
    ws_sz = ctypes.c_size_t(0)
    assert lib.fa_fwd_paged_workspace_size(ctypes.byref(d0), 0, 3, None, None, ctypes.byref(pk()),
                                           ctypes.byref(ws_sz)) == OK
    assert lib.fa_fwd_paged_workspace_size(ctypes.byref(d), 0, 3, None, None, None, ctypes.byref(ws_sz)) == NULLPTR
    assert lib.fa_fwd_paged_workspace_size(ctypes.byref(d), 0, 3, None, None, ctypes.byref(pk(reserved=2)),
                                           ctypes.byref(ws_sz)) == INVALID


def test_fwd_paged_workspace_follows_page_size(lib):
    """Pages of 128 keys keep the 256-row ping-pong tiles (the same workspace as fa_fwd); pages
    of 16 keys fall back to the generic kernel's 64-row tiles, whose work list is longer."""
    buf = (ctypes.c_char * 4096)()
    p = ctypes.cast(buf, ctypes.c_void_p)
    dt = tnd([300, 7], [300, 9])
    qc, kc = [300, 307], [300, 309]
    big = fb.FaPagedKv(p.value, 3, 8, 128, 0, 0)
    small = fb.FaPagedKv(p.value, 19, 64, 16, 1, 0)
    w128 = fb.fa_fwd_paged_workspace_size(dt, "TND", 3, big, qc, kc)
    w16 = fb.fa_fwd_paged_workspace_size(dt, "TND", 3, small, qc, kc)
    assert w128 == fb.fa_fwd_workspace_size(dt, "TND", 3, qc, kc)
    # items (batch, q tile), 8 bytes each: 2 + 1 with 256-row tiles, 5 + 1 with 64-row tiles
    assert w16 - w128 == (6 - 3) * 8
    st = lib.fa_fwd_paged(p, p, p, p, p, ctypes.byref(dt), 2, 3, 0, 0, fb._i64(qc), fb._i64(kc), None, None, 0,
                          None, None, ctypes.byref(small), 0.125, p, w16 - 1, None)
    assert st == WORKSPACE


# ---------------------------------------------------------------------------------------
# Split-KV decode planning (host only)
# ---------------------------------------------------------------------------------------

def _align256(x):
    return (x + 255) // 256 * 256


def test_decode_plan_split_counts(lib):
    """At most 16 query rows per sequence selects the split-KV decode kernel (kernel 3, tiles
    of 16 rows x 64 keys). The split count comes from the launch model (a workgroup costs its
    kv tiles + 3, 256 run at once with D = 128, whole rounds when all are equal, a merge costs
    3, fewer splits win ties within 1%); the values below are worked by hand from that rule.
    work_items counts (batch, split) entries per head; with splits the workspace holds the
    fp32 partial O [slots, N, 16, D] and LSE [slots, N, 16], 256-byte aligned."""
    for B, N, skv, n_split in [
        (1, 1, 333, 1),        # 6 tiles: below one 8-tile split
        (1, 2, 5000, 10),      # 79 tiles, 2 pairs: 10 splits of 8 (est 14) beat 9 of 9 (15)
        (2, 32, 8192, 4),      # 4 x 32 tiles: 256 workgroups in one round (38) beat 8 x 16 (2 rounds, 41)
        (4, 32, 32768, 2),     # 2 x 256 tiles: one round (262) beats one split (515) and 4 x 128 (265)
        (8, 32, 8192, 1),      # 256 pairs of 128 tiles: one round, no merge (131)
        (64, 32, 32768, 1),    # 2048 pairs: no search
    ]:
        d = fb.make_dims(2, 0, B=B, N=N, Sq=1, Skv=skv, D=128)
        st = fb.fa_plan_stats(d, "BNSD", 3)
        assert (st["kernel"], st["block_m"], st["block_n"]) == (3, 16, 64)
        assert st["work_items"] == B * n_split, (B, N, skv, st)
        ws = fb.fa_fwd_workspace_size(d, "BNSD", 3)
        slots = B * N * n_split * 16
        assert ws == (0 if n_split == 1 else _align256(slots * 128 * 4) + _align256(slots * 4)), (B, N, skv)
    # 17 rows, an explicit mask, fp32 or D = 96 stay on the other kernels
    assert fb.fa_plan_stats(fb.make_dims(2, 0, B=1, N=1, Sq=17, Skv=64, D=128), "BNSD", 3)["kernel"] == 1
    assert fb.fa_plan_stats(fb.make_dims(0, 0, B=1, N=1, Sq=1, Skv=64, D=32), "BNSD", 3)["kernel"] == 0
    assert fb.fa_plan_stats(fb.make_dims(2, 0, B=1, N=1, Sq=1, Skv=64, D=96), "BNSD", 3)["kernel"] == 0
    assert fb.fa_plan_stats(fb.make_dims(2, 0, B=1, N=1, Sq=1, Skv=64, D=128), "BNSD", 1,
                            has_mask=True)["kernel"] == 1
    # TND: per-batch splits. Batch 0 (141 tiles) takes 18 splits of 8 tiles; batches 1 (no
    # rows) and 2 (no keys) one entry each and no partial slots. Workspace: geometry (3 x 32
    # bytes), 20 (batch, split) entries, 3 (first slot, splits) pairs, then 18 x 2 slots.
    d = tnd([1, 0, 16], [9000, 5, 0])
    qc, kc = [1, 1, 17], [9000, 9005, 9005]
    st = fb.fa_plan_stats(d, "TND", 3, actual_seq_qlen=qc, actual_seq_kvlen=kc)
    assert st["kernel"] == 3 and st["work_items"] == 20, st
    ws = fb.fa_fwd_workspace_size(d, "TND", 3, qc, kc)
    tables = _align256(_align256(_align256(3 * 32) + 20 * 8) + 3 * 8)
    slots = 18 * 2 * 16
    assert ws == tables + _align256(slots * 128 * 4) + _align256(slots * 4)
    assert st["workspace_bytes"] == ws


# ---------------------------------------------------------------------------------------
# Backward: host validation (no device work)
# ---------------------------------------------------------------------------------------

def test_bwd_validation_and_workspace(lib):
    """fa_bwd applies fa_fwd's argument rules before any launch and needs its own pointers;
    its workspace holds Delta (fp32, laid out like softmax_lse) after the per-batch geometry
    (TND / prefix modes)."""
    buf = (ctypes.c_char * 4096)()
    p = ctypes.cast(buf, ctypes.c_void_p)
    d = bnsd(B=2, N=4, Sq=64, Skv=80, D=128)

    def call(dims=d, mode=3, pre=0, nxt=0, q=p, dq=p, dk=p, lse=p, scale=0.125, ws=p, wsb=4096, alibi_mode=0):
        return lib.fa_bwd(q, p, p, p, lse, p, dq, dk, p, ctypes.byref(dims), 0, mode, pre, nxt, None, None, None,
                          None, alibi_mode, None, None, scale, ws, wsb, None)

    assert call(q=None) == NULLPTR
    assert call(dq=None) == NULLPTR
    assert call(dk=None) == NULLPTR
    assert call(lse=None) == NULLPTR
    assert call(mode=9) == INVALID
    assert call(mode=4, pre=3, nxt=-9) == INVALID
    assert call(scale=0.0) == INVALID
    assert call(alibi_mode=5) == INVALID
    assert call(dims=bnsd(D=129)) == UNSUPPORTED
    need = fb.fa_bwd_workspace_size(d, "BNSD", 3)
    # Delta and the log2-scaled LSE, each laid out like softmax_lse and 256-byte aligned.
    assert need == 2 * _align256(2 * 4 * 64 * 4)
    assert call(wsb=need - 1) == WORKSPACE
    assert call(ws=None, wsb=0) == NULLPTR
    dt = tnd([3, 0, 9], [5, 7, 0])
    need_t = fb.fa_bwd_workspace_size(dt, "TND", 3, [3, 3, 12], [5, 12, 12])
    assert need_t == _align256(3 * 32) + 2 * _align256(2 * 12 * 4)
    # nothing at all to do: OK without pointers
    d0 = bnsd(B=0)
    assert lib.fa_bwd(None, None, None, None, None, None, None, None, None, ctypes.byref(d0), 0, 3, 0, 0, None, None,
                      None, None, 0, None, None, 0.125, None, 0, None) == OK


def test_binding_rejects_mismatched_shapes():
    """The binding checks every shape the C ABI derives from q and k (it has no other way to
    know a buffer's length) before it looks at devices or calls the library: CPU tensors are
    enough to reach each check."""
    import torch

    def t(*shape, dtype=torch.bfloat16):
        return torch.zeros(shape, dtype=dtype)

    B, N, Sq, Skv, D = 2, 3, 5, 7, 16
    q, k, v, o = t(B, N, Sq, D), t(B, N, Skv, D), t(B, N, Skv, D), t(B, N, Sq, D)
    lse = t(B, N, Sq, dtype=torch.float32)
    fb.check_shapes(q, k, v, o, lse, "BNSD")                       # consistent: no error
    bad = [
        dict(v=t(B, N, Skv - 1, D)),                               # short v
        dict(k=t(B, N + 1, Skv, D), v=t(B, N + 1, Skv, D)),        # k heads differ from q
        dict(k=t(B, N, Skv, D + 8), v=t(B, N, Skv, D + 8)),        # k head size differs
        dict(out=t(B, N, Sq - 1, D)),                              # short out
        dict(softmax_lse=t(B, N, Sq - 1, dtype=torch.float32)),    # short lse
        dict(softmax_lse=t(B, Sq, N, dtype=torch.float32)),        # lse not [B, N, Sq]
    ]
    for change in bad:
        args = dict(q=q, k=k, v=v, out=o, softmax_lse=lse)
        args.update(change)
        with pytest.raises(ValueError):
            fb.check_shapes(args["q"], args["k"], args["v"], args["out"], args["softmax_lse"], "BNSD")
        with pytest.raises(ValueError):
            fb.fa_fwd(args["q"], args["k"], args["v"], args["out"], args["softmax_lse"], layout="BNSD",
                      sparse_mode=3, scale=0.25)
    # dense mask: [B | 1, N | 1, Sq, Skv] as mask_bcast says
    m = torch.zeros(B, N, Sq, Skv, dtype=torch.uint8)
    fb.check_shapes(q, k, v, o, lse, "BNSD", atten_mask=m, mask_bcast=[0, 0])
    fb.check_shapes(q, k, v, o, lse, "BNSD", atten_mask=m[:1], mask_bcast=[1, 0])
    fb.check_shapes(q, k, v, o, lse, "BNSD", atten_mask=m[:, :1], mask_bcast=[0, 1])
    for mask, bc in ((m[:, :, :, :-1], [0, 0]), (m[:1], [0, 0]), (m, [1, 0]), (m[:, :1], [1, 1])):
        with pytest.raises(ValueError):
            fb.check_shapes(q, k, v, o, lse, "BNSD", atten_mask=mask, mask_bcast=bc)
        with pytest.raises(ValueError):
            fb.fa_fwd(q, k, v, o, lse, layout="BNSD", sparse_mode=1, scale=0.25, atten_mask=mask,
                      mask_bcast=bc)
    # BSND and TND
    qs, ks = t(B, Sq, N, D), t(B, Skv, N, D)
    fb.check_shapes(qs, ks, ks.clone(), qs.clone(), lse, "BSND")
    with pytest.raises(ValueError):
        fb.check_shapes(qs, ks, t(B, Skv, N - 1, D), qs.clone(), lse, "BSND")
    qt, kt = t(11, N, D), t(13, N, D)
    lt = t(N, 11, dtype=torch.float32)
    fb.check_shapes(qt, kt, kt.clone(), qt.clone(), lt, "TND")
    for args in ((qt, kt, t(12, N, D), qt, lt), (qt, kt, kt, t(10, N, D), lt), (qt, kt, kt, qt, t(11, N, dtype=torch.float32))):
        with pytest.raises(ValueError):
            fb.check_shapes(*args, "TND")
    with pytest.raises(ValueError):
        fb.check_shapes(qt, kt, kt, qt, lt, "TND", atten_mask=torch.zeros(1, 1, 11, 13, dtype=torch.uint8))
    # the backward takes the same checks
    with pytest.raises(ValueError):
        fb.fa_bwd(q, k, t(B, N, Skv - 2, D), o, lse, o.clone(), q.clone(), k.clone(), k.clone(),
                  layout="BNSD", sparse_mode=3, scale=0.25)
    with pytest.raises(ValueError):
        fb.fa_bwd(q, k, v, o, t(B, N, 1, dtype=torch.float32), o.clone(), q.clone(), k.clone(), k.clone(),
                  layout="BNSD", sparse_mode=3, scale=0.25)


def test_noalloc_validates_and_refuses_oversize_before_device_work(lib):
    """fa_fwd_noalloc validates like fa_fwd and refuses a problem whose workspace exceeds
    FA_NOALLOC_SCRATCH_BYTES with FA_ERR_WORKSPACE, all before any HIP call (this host has
    no GPU, so reaching one would fail differently)."""
    buf = (ctypes.c_char * 4096)()
    p = ctypes.cast(buf, ctypes.c_void_p)
    n = 600_000
    ends = list(range(1, n + 1))
    d = tnd([1] * n, [1] * n)
    assert fb.fa_fwd_workspace_size(d, "TND", 3, ends, ends) > fb.FA_NOALLOC_SCRATCH_BYTES
    st = lib.fa_fwd_noalloc(p, p, p, p, p, ctypes.byref(d), 2, 3, 0, 0, fb._i64(ends), fb._i64(ends), None,
                            None, 0, None, None, 0.125, None)
    assert st == WORKSPACE
    st = lib.fa_fwd_noalloc(p, p, p, p, p, ctypes.byref(bnsd()), 0, 4, 3, -9, None, None, None, None, 0, None,
                            None, 0.125, None)
    assert st == INVALID
    st = lib.fa_fwd_noalloc(None, p, p, p, p, ctypes.byref(bnsd()), 0, 3, 0, 0, None, None, None, None, 0, None,
                            None, 0.125, None)
    assert st == NULLPTR


def test_launch_order_choice(lib):
    """The planner's forward launch order (fa_plan_stats.launch_order): rank-major in groups of
    four pairs where item costs spread widely (causal) or come from a mask (mode 1), pair-major
    for bands, batch-major when the (batch, head) pairs do not split over the 8 XCDs, a table for
    varlen and prefix modes, 0 for the decode kernel."""
    def order(dims, layout, mode, **kw):
        return fb.fa_plan_stats(dims, layout, mode, scale=0.088, **kw)["launch_order"]

    big = fb.make_dims(2, 0, B=2, N=32, Sq=8192, Skv=8192, D=128)
    assert order(big, "BNSD", 3) == 3
    assert order(fb.make_dims(2, 0, B=4, N=32, Sq=2048, Skv=2048, D=128), "BNSD", 3) == 3
    assert order(big, "BNSD", 4, pre_tokens=1024, next_tokens=0) == 1
    assert order(big, "BNSD", 0, pre_tokens=1024, next_tokens=-256) == 1
    assert order(big, "BNSD", 1, has_mask=True) == 3
    assert order(fb.make_dims(2, 0, B=1, N=4, Sq=4096, Skv=4096, D=128), "BNSD", 3) == 0
    assert order(big, "BNSD", 5, prefix=[100, 2000]) == 4
    tq = fb.make_dims(2, 2, B=2, N=32, D=128, T_q=3000, T_kv=3000)
    assert order(tq, "TND", 3, actual_seq_qlen=[1000, 3000], actual_seq_kvlen=[1000, 3000]) == 4
    assert order(fb.make_dims(2, 0, B=4, N=32, Sq=1, Skv=32768, D=128), "BNSD", 3) == 0


def test_edge_skip_choice(lib):
    """The planner's ping-pong variant with the empty-wave softmax skip (fa_plan_stats.edge_skip):
    on for bands whose lower bound cuts some row and for items of at most 64 kv tiles; off for
    long causal items (the headline shape), prefix modes, alibi, dense masks and decode."""
    def edge(dims, layout, mode, **kw):
        return fb.fa_plan_stats(dims, layout, mode, scale=0.088, **kw)["edge_skip"]

    big = fb.make_dims(2, 0, B=2, N=32, Sq=8192, Skv=8192, D=128)
    assert edge(big, "BNSD", 3) == 0
    assert edge(fb.make_dims(2, 0, B=4, N=32, Sq=2048, Skv=2048, D=128), "BNSD", 3) == 1
    assert edge(big, "BNSD", 4, pre_tokens=1024, next_tokens=0) == 1
    assert edge(big, "BNSD", 0, pre_tokens=1024, next_tokens=-256) == 1
    assert edge(big, "BNSD", 0, pre_tokens=1 << 30, next_tokens=1 << 30) == 0   # no lower bound
    assert edge(big, "BNSD", 3, has_alibi=True) == 0
    assert edge(big, "BNSD", 1, has_mask=True) == 0
    assert edge(big, "BNSD", 5, prefix=[100, 2000]) == 0
    tq = fb.make_dims(2, 2, B=2, N=32, D=128, T_q=6000, T_kv=6000)
    assert edge(tq, "TND", 3, actual_seq_qlen=[1000, 6000], actual_seq_kvlen=[1000, 6000]) == 0
    t4 = fb.make_dims(2, 2, B=2, N=32, D=128, T_q=5096, T_kv=5096)
    assert edge(t4, "TND", 3, actual_seq_qlen=[1000, 5096], actual_seq_kvlen=[1000, 5096]) == 1
    assert edge(fb.make_dims(2, 0, B=2, N=32, Sq=4097, Skv=4097, D=128), "BNSD", 3) == 0
    assert edge(fb.make_dims(2, 0, B=4, N=32, Sq=1, Skv=32768, D=128), "BNSD", 3) == 0
    assert edge(fb.make_dims(0, 0, B=1, N=1, Sq=64, Skv=64, D=16), "BNSD", 3) == 0   # fp32: generic
