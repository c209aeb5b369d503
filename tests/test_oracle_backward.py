"""Pins for the backward oracle (CPU only): oracle/backward.py against what mathematics fixes
about the derivative of the forward definition, not against itself.

- torch autograd in float64 through an independently written forward (torch softmax and
  matmuls, masks from the oracle's pinned predicate, no use of the backward formulas);
- central finite differences of L = sum(O * dO) on tiny inputs;
- exact invariants: sum_j dK_j = 0 per (batch, head) (each row of dS sums to zero), and
  sum_j dV_j = sum of dO over rows that see a key (each row of P sums to one);
- closed forms: one key per row gives dQ = dK = 0 and dV = sum_i dO_i; an all-masked row
  contributes nothing.
A dropped term of dS, a transposed product or a missing scale fails at least one of them.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle.backward import attention_backward


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _autograd_head(q, k, v, do, vis, scale, bias):
    """Gradients by torch autograd (float64) of the forward written with torch ops."""
    qt, kt, vt = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    s = scale * qt @ kt.T
    if bias is not None:
        s = s + torch.tensor(bias, dtype=torch.float64)
    s = s.masked_fill(~torch.tensor(vis), float("-inf"))
    o = torch.softmax(s, dim=-1) @ vt
    o.backward(torch.tensor(do, dtype=torch.float64))
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


@pytest.mark.parametrize("mode,kw", [(0, dict(pre_tokens=3, next_tokens=2)), (2, {}), (3, {}),
                                     (4, dict(pre_tokens=4, next_tokens=1)), (5, dict(prefix=[3]))])
@pytest.mark.parametrize("alibi", [None, "right", "sqrt", "left"])
def test_matches_float64_autograd(mode, kw, alibi):
    rng = np.random.default_rng(10 + mode)
    sq, skv, D, scale = 7, 9, 5, 0.37
    q, k, v, do = _rand(rng, 1, 1, sq, D), _rand(rng, 1, 1, skv, D), _rand(rng, 1, 1, skv, D), _rand(rng, 1, 1, sq, D)
    slopes = [0.3] if alibi else None
    dq, dk, dv = attention_backward(q, k, v, do, layout="BNSD", sparse_mode=mode, scale=scale, alibi_slopes=slopes,
                                    alibi_mode=alibi or "right", **kw)
    pl = kw.get("prefix", [0])[0]
    vis = oracle.visible_matrix(mode, sq, skv, pre_tokens=kw.get("pre_tokens", 0),
                                next_tokens=kw.get("next_tokens", 0), prefix_len=pl)
    assert vis.any(axis=1).all()   # autograd's softmax needs a visible key in every row
    bias = None
    if alibi:
        bias = oracle.alibi_bias(0.3, np.arange(sq)[:, None], np.arange(skv)[None, :], sq, skv, alibi)
    gq, gk, gv = _autograd_head(q[0, 0], k[0, 0], v[0, 0], do[0, 0], vis, scale, bias)
    np.testing.assert_allclose(dq[0, 0], gq, atol=1e-12, rtol=1e-10)
    np.testing.assert_allclose(dk[0, 0], gk, atol=1e-12, rtol=1e-10)
    np.testing.assert_allclose(dv[0, 0], gv, atol=1e-12, rtol=1e-10)


def test_matches_autograd_dense_mask_and_tnd_split_modes():
    """Mode 1 with a random mask, and the varlen modes 7 / 8 in TND, per (batch, head)."""
    rng = np.random.default_rng(3)
    sq, skv, D = 6, 8, 4
    q, k, v, do = _rand(rng, 2, 2, sq, D), _rand(rng, 2, 2, skv, D), _rand(rng, 2, 2, skv, D), _rand(rng, 2, 2, sq, D)
    mask = (rng.random((2, 2, sq, skv)) < 0.5).astype(np.uint8)
    mask[..., 0] = 0   # every row keeps a visible key
    dq, dk, dv = attention_backward(q, k, v, do, layout="BNSD", sparse_mode=1, scale=0.5, atten_mask=mask)
    for b in range(2):
        for h in range(2):
            g = _autograd_head(q[b, h], k[b, h], v[b, h], do[b, h], mask[b, h] == 0, 0.5, None)
            for mine, ref in zip((dq[b, h], dk[b, h], dv[b, h]), g):
                np.testing.assert_allclose(mine, ref, atol=1e-12, rtol=1e-10)
    ql, kl = [3, 2], [3, 6]     # the pages' split example lengths
    cq, ck = [3, 5], [3, 9]
    q, do = _rand(rng, 5, 2, D), _rand(rng, 5, 2, D)
    k, v = _rand(rng, 9, 2, D), _rand(rng, 9, 2, D)
    for mode, kw in ((7, dict(pre_tokens=6, next_tokens=-4)), (8, dict(pre_tokens=3, next_tokens=0))):
        dq, dk, dv = attention_backward(q, k, v, do, layout="TND", sparse_mode=mode, scale=0.5, actual_seq_qlen=cq,
                                        actual_seq_kvlen=ck, **kw)
        band = oracle.band_batch_index(mode, ql, kl)
        qs, ks = [0, 3], [0, 3]
        for b in range(2):
            vis = oracle.visible_matrix(mode, ql[b], kl[b], band=(b == band), **kw)
            if not vis.any(axis=1).all():
                continue
            for h in range(2):
                g = _autograd_head(q[qs[b]:qs[b] + ql[b], h], k[ks[b]:ks[b] + kl[b], h], v[ks[b]:ks[b] + kl[b], h],
                                   do[qs[b]:qs[b] + ql[b], h], vis, 0.5, None)
                np.testing.assert_allclose(dq[qs[b]:qs[b] + ql[b], h], g[0], atol=1e-12, rtol=1e-10)
                np.testing.assert_allclose(dk[ks[b]:ks[b] + kl[b], h], g[1], atol=1e-12, rtol=1e-10)
                np.testing.assert_allclose(dv[ks[b]:ks[b] + kl[b], h], g[2], atol=1e-12, rtol=1e-10)


def test_finite_differences():
    """dL/dx by central differences of L = sum(O * dO), with O from the forward oracle."""
    rng = np.random.default_rng(5)
    sq, skv, D, scale = 3, 4, 2, 0.8
    q, k, v, do = _rand(rng, 1, 1, sq, D), _rand(rng, 1, 1, skv, D), _rand(rng, 1, 1, skv, D), _rand(rng, 1, 1, sq, D)
    kw = dict(layout="BNSD", sparse_mode=4, scale=scale, pre_tokens=2, next_tokens=0, alibi_slopes=[0.25])

    def loss(q_, k_, v_):
        o, _ = oracle.attention(q_, k_, v_, **kw)
        return float((o * do).sum())

    grads = attention_backward(q, k, v, do, **kw)
    eps = 1e-6
    for which, x in enumerate((q, k, v)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = xp, xm
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        np.testing.assert_allclose(grads[which], num, atol=1e-7, rtol=1e-6)


def test_invariants_dk_sums_to_zero_and_dv_sums_to_do():
    rng = np.random.default_rng(7)
    B, N, sq, skv, D = 2, 3, 11, 13, 6
    q, k, v, do = (_rand(rng, B, N, s, D) for s in (sq, skv, skv, sq))
    for mode, kw in [(3, {}), (0, dict(pre_tokens=2, next_tokens=-1)), (4, dict(pre_tokens=5, next_tokens=0))]:
        dq, dk, dv = attention_backward(q, k, v, do, layout="BNSD", sparse_mode=mode, scale=0.3,
                                        alibi_slopes=[0.1, 0.2, 0.3], **kw)
        np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
        vis = oracle.visible_matrix(mode, sq, skv, **kw)
        live = vis.any(axis=1)
        np.testing.assert_allclose(dv.sum(axis=2), do[:, :, live].sum(axis=2), atol=1e-12)
        # rows that see nothing get no gradient
        assert np.all(dq[:, :, ~live] == 0)


def test_single_key_closed_form():
    """Skv = 1 with leftUpCausal (every row sees key 0): P = 1, so dS = 0 (dQ = dK = 0) and
    dV = sum_i dO_i."""
    rng = np.random.default_rng(9)
    q, do = _rand(rng, 1, 2, 5, 4), _rand(rng, 1, 2, 5, 4)
    k, v = _rand(rng, 1, 2, 1, 4), _rand(rng, 1, 2, 1, 4)
    dq, dk, dv = attention_backward(q, k, v, do, layout="BNSD", sparse_mode=2, scale=1.0)
    assert np.allclose(dq, 0.0, atol=1e-15) and np.allclose(dk, 0.0, atol=1e-15)
    np.testing.assert_allclose(dv[:, :, 0], do.sum(axis=2), atol=1e-14)


def test_layouts_agree():
    """BSND and TND give the BNSD gradients, transposed / packed."""
    rng = np.random.default_rng(11)
    B, N, S, D = 2, 2, 6, 3
    q, k, v, do = (_rand(rng, B, N, S, D) for _ in range(4))
    ref = attention_backward(q, k, v, do, layout="BNSD", sparse_mode=3, scale=0.4)
    t = lambda x: x.transpose(0, 2, 1, 3).copy()
    got = attention_backward(t(q), t(k), t(v), t(do), layout="BSND", sparse_mode=3, scale=0.4)
    for a, b in zip(ref, got):
        np.testing.assert_allclose(t(a), b, atol=1e-14)
    pk = lambda x: x.transpose(0, 2, 1, 3).reshape(B * S, N, D)
    got = attention_backward(pk(q), pk(k), pk(v), pk(do), layout="TND", sparse_mode=3, scale=0.4,
                             actual_seq_qlen=[S, 2 * S], actual_seq_kvlen=[S, 2 * S])
    for a, b in zip(ref, got):
        np.testing.assert_allclose(pk(a), b, atol=1e-14)
