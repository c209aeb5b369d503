"""Plain fp64 CPU oracle for the backward pass of masked attention: dQ, dK and dV.

TEST INFRASTRUCTURE (see the package docstring): only the test suite and the benchmark's
CPU-baseline leg use it.

No page gives a backward pass. This is the derivative of the forward definition in
``oracle.attention`` (the same masks, bias and softmax, one (batch, head) at a time), for a
loss whose gradient with respect to O is dO:

    S = scale * Q K^T + bias,   S[masked] = -inf,   P = softmax_rows(S),   O = P V
    dV = P^T dO
    dP = dO V^T
    dS = P * (dP - rowsum(P * dP))          (the softmax Jacobian applied row by row)
    dQ = scale * dS K
    dK = scale * dS^T Q

Masked entries have P = 0 and therefore dS = 0; a row with no visible key (O = 0 by the
forward's convention) contributes nothing to any gradient. The alibi bias and the mask are
constants: they enter only through P. Every value is float64.
"""

from __future__ import annotations

import numpy as np

from .attention import (_dims, _head_view, _mask_rows, _segments, alibi_bias, band_batch_index,
                        visible)


def attention_head_backward(q, k, v, do, vis, scale: float, bias=None):
    """(dq, dk, dv) for one (batch, head): q, do [R, D]; k, v [Skv, D]; vis [R, Skv]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    rows = q.shape[0]
    s = float(scale) * (q @ k.T)
    if bias is not None:
        s = s + bias
    s = np.where(vis, s, -np.inf)
    p = np.zeros_like(s)
    live = vis.any(axis=1) if vis.shape[1] else np.zeros(rows, dtype=bool)
    if live.any():
        sl = s[live]
        e = np.exp(sl - sl.max(axis=1, keepdims=True))
        p[live] = e / e.sum(axis=1, keepdims=True)
    dv = p.T @ do
    dp = do @ v.T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    dq = float(scale) * (ds @ k)
    dk = float(scale) * (ds.T @ q)
    return dq, dk, dv


def attention_backward(q, k, v, do, *, layout: str = "BNSD", sparse_mode: int = 0, scale: float,
                       pre_tokens: int = 0, next_tokens: int = 0, actual_seq_qlen=None,
                       actual_seq_kvlen=None, prefix=None, alibi_slopes=None, atten_mask=None,
                       alibi_mode: str = "right"):
    """Gradients of the full forward pass (same arguments as ``oracle.attention`` plus dO in
    q's layout). Returns (dq, dk, dv) in the layouts of q, k and v."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    n, sq, skv = _dims(layout, q, k)
    segs = _segments(layout, q, k, sq, skv, actual_seq_qlen, actual_seq_kvlen)
    band_b = band_batch_index(sparse_mode, [s[1] for s in segs], [s[3] for s in segs])
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b, (qs, ql, ks, kl) in enumerate(segs):
        pl = int(prefix[b]) if prefix is not None else 0
        for h in range(n):
            rows = np.arange(ql)
            kw = dict(pre_tokens=pre_tokens, next_tokens=next_tokens, prefix_len=pl, band=(b == band_b))
            if sparse_mode == 1:
                kw["mask_rows"] = _mask_rows(atten_mask, b, h, rows, kl)
            vis = np.broadcast_to(visible(sparse_mode, rows[:, None], np.arange(kl)[None, :], ql, kl, **kw),
                                  (ql, kl))
            bias = None
            if alibi_slopes is not None:
                bias = alibi_bias(alibi_slopes[h], rows[:, None], np.arange(kl)[None, :], ql, kl, alibi_mode)
            g = attention_head_backward(_head_view(q, layout, b, h, qs, ql), _head_view(k, layout, b, h, ks, kl),
                                        _head_view(v, layout, b, h, ks, kl), _head_view(do, layout, b, h, qs, ql),
                                        vis, scale, bias)
            for dst, src, start, length in ((dq, g[0], qs, ql), (dk, g[1], ks, kl), (dv, g[2], ks, kl)):
                if layout == "BNSD":
                    dst[b, h, :length] = src
                elif layout == "BSND":
                    dst[b, :length, h] = src
                else:
                    dst[start:start + length, h] = src
    return dq, dk, dv
