"""Pins for the fp64 oracle, checked against what the pages and mathematics fix (CPU only).

Each test names the passage it follows. None of them re-types the oracle's own formula:
they use the pages' worked examples, hand-derived intervals, closed forms, library routines
(torch's softmax / scaled_dot_product_attention / logsumexp in float64) and invariants
the page text implies.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from masked_attention_forward_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(1234)


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------------------
# Masks
# ---------------------------------------------------------------------------------------

def _valid_band(sq, skv, rng):
    """Random (pre, next) satisfying the page's sign constraints for mode 0."""
    while True:
        pre = int(rng.integers(-sq, sq + 4))
        nxt = int(rng.integers(-skv, skv + 4))
        if nxt < 0 and not (pre >= -nxt and -nxt < max(skv, 1)):
            continue
        if pre < 0 and not (nxt >= -pre and -pre < max(sq, 1)):
            continue
        return pre, nxt


@pytest.mark.parametrize("mode", [0, 1, 2, 3, 4, 5, 6, 7, 8])
def test_predicate_matches_loop_enumeration(mode):
    """Vectorised predicate == nested-loop enumeration, on random tiny shapes."""
    rng = np.random.default_rng(100 + mode)
    for _ in range(40):
        sq = int(rng.integers(0, 24))
        skv = int(rng.integers(0, 24))
        pre, nxt = _valid_band(sq, skv, rng)
        pl = int(rng.integers(0, skv + 2))
        band = bool(rng.integers(0, 2))
        mask = rng.integers(0, 2, size=(sq, skv)).astype(np.uint8)
        kw = dict(pre_tokens=pre, next_tokens=nxt, prefix_len=pl, band=band)
        if mode == 1:
            vis = oracle.visible(1, np.arange(sq)[:, None], np.arange(skv)[None, :], sq, skv,
                                 mask_rows=mask)
            vis = np.broadcast_to(vis, (sq, skv))
        else:
            vis = oracle.visible_matrix(mode, sq, skv, **kw)
        loops = oracle.count_visible_loops(mode, sq, skv, mask=mask, **kw)
        assert list(vis.sum(axis=1)) == loops


def test_band_examples_hand_derived():
    """sparseMode介绍, sparseMode=0: pre=9/next=-3 and next=7/pre=-3 on 16x16."""
    g = _load("band_examples.json")
    for case in g["cases"]:
        vis = oracle.visible_matrix(0, case["sq"], case["skv"], pre_tokens=case["pre_tokens"],
                                    next_tokens=case["next_tokens"])
        assert int(vis.sum()) == case["total"]
        assert list(vis.sum(axis=1)) == case["counts"]
        for i, iv in enumerate(case["rows"]):
            cols = np.nonzero(vis[i])[0]
            if iv is None:
                assert cols.size == 0
            else:
                assert cols.tolist() == list(range(iv[0], iv[1] + 1))


def test_mode0_causal_reading():
    """sparseMode=0 with nextTokens=0 and preTokens >= Sq is the causal case (lower triangle
    with the diagonal), i.e. the same mask as leftUpCausal (sparseMode=2)."""
    for sq, skv in [(5, 5), (7, 9), (9, 4), (1, 1)]:
        a = oracle.visible_matrix(0, sq, skv, pre_tokens=sq, next_tokens=0)
        b = oracle.visible_matrix(2, sq, skv)
        assert np.array_equal(a, b)
        assert np.array_equal(b, np.tril(np.ones((sq, skv), dtype=bool)))


def test_right_down_causal_closed_form():
    """sparseMode=3 (origin at the bottom-right vertex): for Sq <= Skv every row is
    non-empty and the total is Sq*(Skv-Sq) + Sq*(Sq+1)/2; the last row sees every key."""
    for sq, skv in [(4, 6), (3, 3), (4096 // 64, 8192 // 64), (1, 7)]:
        vis = oracle.visible_matrix(3, sq, skv)
        assert int(vis.sum()) == sq * (skv - sq) + sq * (sq + 1) // 2
        assert vis[-1].all()
        assert np.array_equal(vis, np.tri(sq, skv, k=skv - sq, dtype=bool))


@pytest.mark.parametrize("which", ["mode7", "mode8"])
def test_split_examples_rows_equal_unsplit(which):
    """sparseMode=7 / 8 worked examples: the two cards' rows equal the unsplit rows, both
    the visible pattern (exactly) and O / LSE (to fp64 rounding), with the same K and V."""
    ex = _load("split_examples.json")[which]
    un = ex["unsplit"]
    d = 8
    rng = np.random.default_rng(7 if which == "mode7" else 8)
    qlens, kvlens = un["qlens"], un["kvlens"]
    qs_un = [rng.standard_normal((n, 1, d)) for n in qlens]
    ks_un = [rng.standard_normal((n, 1, d)) for n in kvlens]
    vs_un = [rng.standard_normal((n, 1, d)) for n in kvlens]
    cq = synth.cumulative_ends(qlens)
    ck = synth.cumulative_ends(kvlens)
    o_un, l_un = oracle.attention(np.concatenate(qs_un), np.concatenate(ks_un),
                                  np.concatenate(vs_un), layout="TND",
                                  sparse_mode=un["sparse_mode"], scale=0.3,
                                  actual_seq_qlen=cq, actual_seq_kvlen=ck)
    starts_un = [0] + cq[:-1]
    for card in ("card1", "card2"):
        c = ex[card]
        qcum, kcum = c["actual_seq_qlen"], c["actual_seq_kvlen"]
        q_parts, k_parts, v_parts = [], [], []
        for (ub, r0, nrows) in c["unsplit_rows"]:
            q_parts.append(qs_un[ub][r0:r0 + nrows])
            k_parts.append(ks_un[ub])
            v_parts.append(vs_un[ub])
        # the page's cumulative arrays must describe exactly these shard shapes
        assert synth.cumulative_ends([p.shape[0] for p in q_parts]) == qcum
        assert synth.cumulative_ends([p.shape[0] for p in k_parts]) == kcum
        o_c, l_c = oracle.attention(np.concatenate(q_parts), np.concatenate(k_parts),
                                    np.concatenate(v_parts), layout="TND",
                                    sparse_mode=c["sparse_mode"], scale=0.3,
                                    pre_tokens=c["pre_tokens"], next_tokens=c["next_tokens"],
                                    actual_seq_qlen=qcum, actual_seq_kvlen=kcum)
        band_b = oracle.band_batch_index(c["sparse_mode"], np.diff([0] + qcum), np.diff([0] + kcum))
        row = 0
        for b, (ub, r0, nrows) in enumerate(c["unsplit_rows"]):
            sq_c, skv_c = nrows, kvlens[ub]
            vis_c = oracle.visible_matrix(c["sparse_mode"], sq_c, skv_c,
                                          pre_tokens=c["pre_tokens"],
                                          next_tokens=c["next_tokens"], band=(b == band_b))
            vis_u = oracle.visible_matrix(un["sparse_mode"], qlens[ub], kvlens[ub])
            assert np.array_equal(vis_c, vis_u[r0:r0 + nrows])
            src = starts_un[ub] + r0
            np.testing.assert_allclose(o_c[row:row + nrows], o_un[src:src + nrows], atol=1e-13)
            np.testing.assert_allclose(l_c[:, row:row + nrows], l_un[:, src:src + nrows],
                                       atol=1e-13)
            row += nrows


def test_split_example_pins_inclusive_next_and_right_down_origin():
    """The mode-7 example fails under the two nearby readings: an exclusive nextTokens bound
    or a top-left origin for the band batch would not reproduce unsplit rows 0-1."""
    un = oracle.visible_matrix(3, 4, 6)[0:2]
    good = oracle.visible_matrix(7, 2, 6, pre_tokens=6, next_tokens=-2, band=True)
    assert np.array_equal(good, un)
    top_left = oracle.visible_matrix(0, 2, 6, pre_tokens=6, next_tokens=-2)
    assert not np.array_equal(top_left, un)
    exclusive = oracle.visible_matrix(7, 2, 6, pre_tokens=6, next_tokens=-3, band=True)
    assert not np.array_equal(exclusive, un)


def test_prefix_mode_edges():
    """sparseMode=5/6: prefix columns are counted from the left; prefix <= off+1 adds
    nothing to rightDownCausal and prefix = Skv opens every column."""
    for sq, skv in [(6, 6), (4, 9), (7, 3)]:
        off = skv - sq
        lim = max(off + 1, 0)          # row 0 already sees columns 0 .. off
        c3 = oracle.visible_matrix(3, sq, skv)
        for pl in range(0, lim + 1):
            assert np.array_equal(oracle.visible_matrix(5, sq, skv, prefix_len=pl), c3)
        if lim + 1 <= skv:
            more = oracle.visible_matrix(5, sq, skv, prefix_len=lim + 1)
            assert more.sum() > c3.sum()
            assert more[0, lim] and not c3[0, lim]
        assert oracle.visible_matrix(5, sq, skv, prefix_len=skv).all()
        assert np.array_equal(oracle.visible_matrix(6, sq, skv, prefix_len=3),
                              oracle.visible_matrix(5, sq, skv, prefix_len=3))


def test_band_modes_equivalences():
    """sparseMode=4 with next=0 and pre covering everything is rightDownCausal; mode 2 and
    mode 3 coincide when Sq = Skv; mode 7 with one batch is the band rule itself."""
    for sq, skv in [(5, 5), (4, 9), (9, 4)]:
        assert np.array_equal(oracle.visible_matrix(4, sq, skv, pre_tokens=sq + skv, next_tokens=0),
                              oracle.visible_matrix(3, sq, skv))
    assert np.array_equal(oracle.visible_matrix(2, 6, 6), oracle.visible_matrix(3, 6, 6))
    assert oracle.band_batch_index(7, [5], [9]) == 0
    assert oracle.band_batch_index(8, [0, 3, 2], [4, 5, 0]) == 1
    assert oracle.band_batch_index(7, [0, 3, 2, 0], [4, 5, 1, 3]) == 2


# ---------------------------------------------------------------------------------------
# Softmax, LSE and the recurrence
# ---------------------------------------------------------------------------------------

@pytest.mark.parametrize("example,block", [(1, 4), (2, 3)])
def test_page_examples_tiled_equals_naive(example, block):
    """Exercise page, examples 1 and 2: the tiled recurrence equals softmax(q k^T / sqrt(D)) v
    computed with torch in float64, and so does the dense definition."""
    q, k, v = synth.page_example_tensors(example)
    d = q.shape[-1]
    scores = torch.matmul(q, k.transpose(-2, -1)) / math.sqrt(d)
    ref = torch.matmul(torch.softmax(scores, dim=-1), v).numpy()
    ref_lse = torch.logsumexp(scores, dim=-1).numpy()
    o_t, l_t = oracle.tiled_attention(q.numpy(), k.numpy(), v.numpy(), block_size=block)
    assert o_t.shape == tuple(q.shape)
    np.testing.assert_allclose(o_t, ref, atol=1e-12, rtol=0)
    np.testing.assert_allclose(l_t, ref_lse, atol=1e-12, rtol=0)
    o_d, l_d = oracle.attention(q.unsqueeze(1).numpy(), k.unsqueeze(1).numpy(),
                                v.unsqueeze(1).numpy(), layout="BNSD", sparse_mode=0,
                                scale=1 / math.sqrt(d), pre_tokens=synth.NO_MASK,
                                next_tokens=synth.NO_MASK)
    np.testing.assert_allclose(o_d[:, 0], ref, atol=1e-12, rtol=0)
    np.testing.assert_allclose(l_d[:, 0], ref_lse, atol=1e-12, rtol=0)


def _sdpa_ref(q, k, v, vis, scale, bias=None):
    """torch SDPA (float64, CPU) with a boolean attend-mask or an additive float mask."""
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(x))[None, None] for x in (q, k, v))
    if bias is None:
        m = torch.from_numpy(vis)[None, None]
    else:
        m = torch.from_numpy(np.where(vis, bias, -np.inf))[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    s = scale * (torch.from_numpy(q) @ torch.from_numpy(k).T)
    s = s + (torch.from_numpy(bias) if bias is not None else 0)
    s = s.masked_fill(~torch.from_numpy(vis), float("-inf"))
    return o[0, 0].numpy(), torch.logsumexp(s, dim=-1).numpy()


@pytest.mark.parametrize("mode", [0, 1, 2, 3, 4, 5, 7, 8])
@pytest.mark.parametrize("with_bias", [False, True])
def test_head_matches_torch_sdpa(mode, with_bias):
    """attention_head == torch scaled_dot_product_attention (float64) on rows that are not
    fully masked, with the mask built by the oracle's predicate; LSE == torch.logsumexp."""
    rng = np.random.default_rng(200 + mode)
    for sq, skv, d in [(7, 11, 8), (13, 5, 16), (9, 9, 4)]:
        q = rng.standard_normal((sq, d))
        k = rng.standard_normal((skv, d))
        v = rng.standard_normal((skv, d))
        pre, nxt = _valid_band(sq, skv, rng)
        kw = dict(pre_tokens=pre, next_tokens=nxt, prefix_len=3, band=True)
        if mode == 1:
            mask = rng.integers(0, 2, size=(sq, skv)).astype(np.uint8)
            vis = np.broadcast_to(oracle.visible(1, np.arange(sq)[:, None], np.arange(skv)[None, :],
                                                 sq, skv, mask_rows=mask), (sq, skv))
        else:
            vis = oracle.visible_matrix(mode, sq, skv, **kw)
        bias = None
        if with_bias:
            bias = oracle.alibi_bias(0.37, np.arange(sq)[:, None], np.arange(skv)[None, :], sq, skv)
        o, lse = oracle.attention_head(q, k, v, vis, 0.41, bias)
        live = vis.any(axis=1)
        if live.any():
            ref_o, ref_lse = _sdpa_ref(q, k, v, np.ascontiguousarray(vis), 0.41, bias)
            np.testing.assert_allclose(o[live], ref_o[live], atol=1e-12, rtol=0)
            np.testing.assert_allclose(lse[live], ref_lse[live], atol=1e-12, rtol=0)
        assert np.all(o[~live] == 0.0)
        assert np.all(np.isneginf(lse[~live]))


def test_closed_form_identical_keys():
    """All keys equal: O_i = mean of the visible v_j; LSE_i = scale q_i.k + ln(count_i)."""
    sq, skv, d = 9, 14, 8
    rng = np.random.default_rng(3)
    q = rng.standard_normal((sq, d))
    k = np.tile(rng.standard_normal((1, d)), (skv, 1))
    v = rng.standard_normal((skv, d))
    vis = oracle.visible_matrix(4, sq, skv, pre_tokens=3, next_tokens=1)
    o, lse = oracle.attention_head(q, k, v, vis, 0.5)
    for i in range(sq):
        n = int(vis[i].sum())
        if n == 0:
            continue
        np.testing.assert_allclose(o[i], v[vis[i]].mean(axis=0), atol=1e-13)
        np.testing.assert_allclose(lse[i], 0.5 * q[i] @ k[0] + math.log(n), atol=1e-13)


def test_closed_form_alibi_geometric_lse():
    """q = 0 with alibi on right-down causal rows: the scores are slope * (j - i - off) for
    j <= i + off, a geometric series: LSE_i = ln((1 - e^{-s n_i}) / (1 - e^{-s})) with
    n_i = i + off + 1. Fixes the bias sign and its bottom-right alignment."""
    sq, skv, d, slope = 6, 10, 4, 0.3
    off = skv - sq
    q = np.zeros((sq, d))
    rng = np.random.default_rng(5)
    k = rng.standard_normal((skv, d))
    v = rng.standard_normal((skv, d))
    vis = oracle.visible_matrix(3, sq, skv)
    bias = oracle.alibi_bias(slope, np.arange(sq)[:, None], np.arange(skv)[None, :], sq, skv)
    _, lse = oracle.attention_head(q, k, v, vis, 0.7, bias)
    for i in range(sq):
        n = i + off + 1
        ref = math.log((1 - math.exp(-slope * n)) / (1 - math.exp(-slope)))
        assert abs(lse[i] - ref) < 1e-13


def test_single_visible_key_returns_that_value():
    """A row with exactly one visible key returns that key's value row."""
    sq, skv, d = 5, 5, 6
    rng = np.random.default_rng(9)
    q, k, v = (rng.standard_normal((n, d)) for n in (sq, skv, skv))
    vis = oracle.visible_matrix(0, sq, skv, pre_tokens=0, next_tokens=0)   # the diagonal only
    o, lse = oracle.attention_head(q, k, v, vis, 0.9)
    np.testing.assert_array_equal(o, v)
    np.testing.assert_allclose(lse, 0.9 * np.einsum("id,id->i", q, k), atol=1e-13)


def test_fully_masked_rows_convention():
    """Reading for rows with nothing visible (mode 0 with next < 0 leaves the first |next|
    rows empty): O = 0 and LSE = -inf, in both the definition and the recurrence."""
    sq = skv = 16
    rng = np.random.default_rng(11)
    q, k, v = (rng.standard_normal((1, sq, 8)) for _ in range(3))
    vis = oracle.visible_matrix(0, sq, skv, pre_tokens=9, next_tokens=-3)
    o, lse = oracle.attention_head(q[0], k[0], v[0], vis, 0.35)
    assert np.all(o[:3] == 0) and np.all(np.isneginf(lse[:3]))
    o_t, l_t = oracle.tiled_attention(q, k, v, block_size=4, scale=0.35, vis=vis[None])
    np.testing.assert_allclose(o_t[0], o, atol=1e-13)
    assert np.all(np.isneginf(l_t[0, :3]))
    np.testing.assert_allclose(l_t[0, 3:], lse[3:], atol=1e-13)


@pytest.mark.parametrize("mode", [0, 3, 4, 5])
def test_tiled_recurrence_with_mask_and_bias(mode):
    """The page's recurrence with masking and a bias equals the dense definition, with a
    block size that leaves ragged tails."""
    rng = np.random.default_rng(300 + mode)
    sq, skv, d = 11, 17, 8
    q, k, v = rng.standard_normal((1, sq, d)), rng.standard_normal((1, skv, d)), rng.standard_normal((1, skv, d))
    vis = oracle.visible_matrix(mode, sq, skv, pre_tokens=4, next_tokens=2, prefix_len=9)
    bias = oracle.alibi_bias(0.21, np.arange(sq)[:, None], np.arange(skv)[None, :], sq, skv)
    o_d, l_d = oracle.attention_head(q[0], k[0], v[0], vis, 0.3, bias)
    o_t, l_t = oracle.tiled_attention(q, k, v, 5, scale=0.3, vis=vis[None], bias=bias[None])
    np.testing.assert_allclose(o_t[0], o_d, atol=1e-12)
    live = vis.any(axis=1)
    np.testing.assert_allclose(l_t[0, live], l_d[live], atol=1e-12)


def test_alibi_left_vs_right_alignment_shift():
    """Shifting the bias by a per-row constant leaves O unchanged and moves LSE by that
    constant: right-aligned vs left-aligned bias differ by slope * (Skv - Sq)."""
    sq, skv, d, slope = 5, 9, 4, 0.25
    rng = np.random.default_rng(4)
    q, k, v = (rng.standard_normal((n, d)) for n in (sq, skv, skv))
    vis = oracle.visible_matrix(3, sq, skv)
    i, j = np.arange(sq)[:, None], np.arange(skv)[None, :]
    right = oracle.alibi_bias(slope, i, j, sq, skv)
    left = slope * (j - i).astype(np.float64)
    o_r, l_r = oracle.attention_head(q, k, v, vis, 0.5, right)
    o_l, l_l = oracle.attention_head(q, k, v, vis, 0.5, left)
    np.testing.assert_allclose(o_r, o_l, atol=1e-13)
    np.testing.assert_allclose(l_l - l_r, slope * (skv - sq), atol=1e-13)


def test_alibi_left_mode_is_a_row_shift_of_right():
    """"压缩mask", alibi scenario, left-aligned vs right-aligned bias: per row the two differ
    by the constant slope * (Skv - Sq), so O is the same and LSE moves by that constant,
    per head, whatever the mask (modes 3 and 5, Sq != Skv)."""
    rng = np.random.default_rng(41)
    B, N, sq, skv, d = 2, 3, 6, 11, 8
    q, k, v = (rng.standard_normal((B, N, n, d)) for n in (sq, skv, skv))
    slopes = [0.5, 0.25, 0.125]
    for mode, extra in ((3, {}), (5, {"prefix": [9, 2]})):
        o_r, l_r = oracle.attention(q, k, v, sparse_mode=mode, scale=0.3, alibi_slopes=slopes, **extra)
        o_l, l_l = oracle.attention(q, k, v, sparse_mode=mode, scale=0.3, alibi_slopes=slopes,
                                    alibi_mode="left", **extra)
        np.testing.assert_allclose(o_l, o_r, atol=1e-13)
        for h, sl in enumerate(slopes):
            np.testing.assert_allclose(l_l[:, h] - l_r[:, h], sl * (skv - sq), atol=1e-12)


def _one_hot_probe(sq, skv, mode, slope, alibi_mode, **kw):
    """q = 0 and v = identity: O_i is the row's softmax weight vector, LSE_i its log-sum."""
    q = np.zeros((1, 1, sq, 4))
    k = np.ones((1, 1, skv, 4))
    v = np.eye(skv)[None, None]
    return oracle.attention(q, k, v, sparse_mode=mode, scale=1.0, alibi_slopes=[slope],
                            alibi_mode=alibi_mode, **kw)


def test_alibi_sqrt_closed_form_causal():
    """"压缩mask", alibi scenario, square-root right-aligned bias: with q = 0 the score of key
    j in right-down causal row i is -slope * sqrt(d), d = i + (Skv - Sq) - j >= 0, so
    LSE_i = ln sum_{d=0}^{i+off} exp(-slope sqrt(d)) and the weights are exp(-slope sqrt(d) - LSE_i)
    (closed form evaluated here with math.fsum)."""
    sq, skv, slope = 5, 9, 0.7
    off = skv - sq
    o, lse = _one_hot_probe(sq, skv, 3, slope, "sqrt")
    for i in range(sq):
        ds = [i + off - j for j in range(i + off + 1)]
        ref_lse = math.log(math.fsum(math.exp(-slope * math.sqrt(dd)) for dd in ds))
        assert abs(lse[0, 0, i] - ref_lse) < 1e-12
        for j in range(skv):
            w = math.exp(-slope * math.sqrt(i + off - j) - ref_lse) if j <= i + off else 0.0
            assert abs(o[0, 0, i, j] - w) < 1e-12


def test_alibi_sqrt_above_diagonal_sign():
    """Keys right of the bottom-right diagonal (visible in a mode-4 band with next > 0) get the
    positive bias slope * sqrt(j - i - off): the reading that keeps the right-aligned bias's
    sign and square-roots its magnitude."""
    sq, skv, slope = 4, 6, 0.5
    off = skv - sq
    o, lse = _one_hot_probe(sq, skv, 4, slope, "sqrt", pre_tokens=1, next_tokens=2)
    above = 0
    for i in range(sq):
        js = [j for j in range(skv) if -1 <= j - i - off <= 2]
        sc = {j: -slope * math.copysign(math.sqrt(abs(i + off - j)), i + off - j) for j in js}
        ref_lse = math.log(math.fsum(math.exp(x) for x in sc.values()))
        assert abs(lse[0, 0, i] - ref_lse) < 1e-12
        for j in js:
            assert abs(o[0, 0, i, j] - math.exp(sc[j] - ref_lse)) < 1e-12
        above += sum(j > i + off for j in js)
    assert above > 0


def test_alibi_zero_slope_is_no_bias():
    """A zero slope leaves every variant equal to attention without alibi."""
    rng = np.random.default_rng(43)
    q, k, v = (rng.standard_normal((1, 2, n, 8)) for n in (5, 7, 7))
    o0, l0 = oracle.attention(q, k, v, sparse_mode=3, scale=0.4)
    for m in oracle.ALIBI_MODES:
        o, l = oracle.attention(q, k, v, sparse_mode=3, scale=0.4, alibi_slopes=[0.0, 0.0], alibi_mode=m)
        np.testing.assert_allclose(o, o0, atol=1e-14)
        np.testing.assert_allclose(l, l0, atol=1e-14)


# ---------------------------------------------------------------------------------------
# Layouts
# ---------------------------------------------------------------------------------------

def test_layouts_agree():
    """BNSD == BSND after a transpose; TND with equal lengths == BSND."""
    rng = np.random.default_rng(21)
    B, N, S, D = 3, 2, 7, 8
    q, k, v = (rng.standard_normal((B, N, S, D)) for _ in range(3))
    o1, l1 = oracle.attention(q, k, v, layout="BNSD", sparse_mode=3, scale=0.4)
    tr = lambda x: np.ascontiguousarray(x.transpose(0, 2, 1, 3))
    o2, l2 = oracle.attention(tr(q), tr(k), tr(v), layout="BSND", sparse_mode=3, scale=0.4)
    np.testing.assert_allclose(tr(o2), o1, atol=1e-14)
    np.testing.assert_allclose(l2, l1, atol=1e-14)
    flat = lambda x: tr(x).reshape(B * S, N, D)
    cum = synth.cumulative_ends([S] * B)
    o3, l3 = oracle.attention(flat(q), flat(k), flat(v), layout="TND", sparse_mode=3, scale=0.4,
                              actual_seq_qlen=cum, actual_seq_kvlen=cum)
    np.testing.assert_allclose(o3, flat(o1), atol=1e-14)
    np.testing.assert_allclose(l3, l1.transpose(1, 0, 2).reshape(N, B * S), atol=1e-14)


def test_rows_match_full():
    """attention_rows gives the same rows as the full evaluation (alibi, prefix, TND)."""
    rng = np.random.default_rng(22)
    lens, kl = [5, 9, 3], [7, 9, 6]
    N, D = 2, 8
    q = rng.standard_normal((sum(lens), N, D))
    k = rng.standard_normal((sum(kl), N, D))
    v = rng.standard_normal((sum(kl), N, D))
    kw = dict(layout="TND", sparse_mode=5, scale=0.3, actual_seq_qlen=synth.cumulative_ends(lens),
              actual_seq_kvlen=synth.cumulative_ends(kl), prefix=[2, 6, 0], alibi_slopes=[0.5, 0.25])
    o, lse = oracle.attention(q, k, v, **kw)
    rows = [(0, 1, 4), (1, 0, 0), (2, 1, 2), (1, 1, 8)]
    o_r, l_r = oracle.attention_rows(q, k, v, rows, **kw)
    starts = [0, 5, 14]
    for r, (b, h, i) in enumerate(rows):
        np.testing.assert_allclose(o_r[r], o[starts[b] + i, h], atol=1e-14)
        np.testing.assert_allclose(l_r[r], lse[h, starts[b] + i], atol=1e-14)


def test_mode1_mask_of_another_mode_is_that_mode():
    """sparseMode=1 fed the boolean mask (True = masked) of mode k gives mode k's result."""
    rng = np.random.default_rng(23)
    B, N, S, D = 2, 2, 9, 8
    q, k, v = (rng.standard_normal((B, N, S, D)) for _ in range(3))
    for mode, extra in [(3, {}), (4, dict(pre_tokens=2, next_tokens=1)), (0, dict(pre_tokens=9, next_tokens=-3))]:
        vis = oracle.visible_matrix(mode, S, S, **extra)
        mask = (~vis).astype(np.uint8)[None, None]
        o1, l1 = oracle.attention(q, k, v, sparse_mode=1, scale=0.3, atten_mask=mask)
        ok, lk = oracle.attention(q, k, v, sparse_mode=mode, scale=0.3, **extra)
        np.testing.assert_allclose(o1, ok, atol=1e-14)
        np.testing.assert_array_equal(np.isneginf(l1), np.isneginf(lk))
        fin = np.isfinite(lk)
        np.testing.assert_allclose(l1[fin], lk[fin], atol=1e-14)
