"""Plain fp64 CPU oracle for masked scaled-dot-product attention forward.

TEST INFRASTRUCTURE. Only the test suite, the smoke entry point and the benchmark's
CPU-baseline leg may import or call this module. The product library never does, and this
module imports nothing from it: the two share no code.

What it computes is the plain definition, written out so it can be checked by eye against
the pages:

    S = scale * Q K^T + bias,   S[masked] = -inf,   P = softmax_rows(S),   O = P V,
    LSE_i = log(sum_j exp(S_ij)) over the visible j of row i.

The full Sq x Skv score matrix and an explicit boolean mask are materialised per
(batch, head). Every value is float64.

Sources (cited by page title and section):
- "sparseMode介绍" (CANN aolapi, common parameter page): the attenMask convention (True =
  the QK^T entry is masked) and the definitions of sparseMode 0..8 in the sections
  "sparseMode=0" .. "sparseMode=8", with the worked split examples of modes 7 and 8.
- "压缩mask" (CANN ATB, compressed mask page), section "不同压缩mask的构造方法", alibi
  scenario: the alibi mask is a per-head coefficient (slope) times a relative-position bias
  plus the triangular mask; the bias is right-aligned; the operator aligns masks from
  kvSeqLen and qSeqLen.
- "Ý Tưởng Tiling & Online Softmax Trong FlashAttention" (exercise page), section "Mục tiêu
  kiến thức": block tiling and the running max / running sum recurrence, implemented in
  :func:`tiled_attention` as a second, independent code path.

Readings taken where the pages are silent or garbled (all listed in the design notes):
- mode 0 measures offsets from the top-left corner (j - i); modes 4, 7 and 8 (band batch)
  from the bottom-right corner (j - i - (Skv - Sq)).
- both band bounds are inclusive.
- a row whose every key is masked yields O = 0 and LSE = -inf.
- the alibi bias is added after scaling. Right-aligned: slope_h * (j - i - (Skv - Sq));
  the square-root variant takes the square root of that bias's magnitude (sign kept);
  left-aligned: slope_h * (j - i). The page's figures with the exact values are missing.
- modes 5 and 6: columns j < prefix_b are visible in addition to right-down causal.
- modes 7 and 8: the band batch is the last (7) or first (8) batch with Sq_b > 0 and
  Skv_b > 0.
"""

from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence

import numpy as np

LAYOUTS = ("BNSD", "BSND", "TND")


# ----------------------------------------------------------------------------------------
# Masks: the literal per-mode predicates ("sparseMode介绍", sections sparseMode=0..8).
# ----------------------------------------------------------------------------------------

def band_batch_index(sparse_mode: int, qlens: Sequence[int], kvlens: Sequence[int]) -> Optional[int]:
    """Index of the batch that carries the band mask in sparseMode 7 / 8, else None.

    "sparseMode介绍", sections sparseMode=7 and sparseMode=8 (notes): in mode 7 the band
    applies to the last batch whose tensor is non-empty, in mode 8 to the first one.
    Non-empty is read as Sq_b > 0 and Skv_b > 0.
    """
    if sparse_mode not in (7, 8):
        return None
    nonempty = [b for b in range(len(qlens)) if qlens[b] > 0 and kvlens[b] > 0]
    if not nonempty:
        return None
    return nonempty[-1] if sparse_mode == 7 else nonempty[0]


def visible(sparse_mode: int, i, j, sq: int, skv: int, *, pre_tokens: int = 0,
            next_tokens: int = 0, prefix_len: int = 0, band: bool = False,
            mask_rows=None) -> np.ndarray:
    """Boolean "visible" (not masked) for query rows ``i`` and key columns ``j``.

    ``i`` and ``j`` are broadcastable integer arrays of batch-local positions. The rules
    follow "sparseMode介绍", one section per mode:

    - 0 (defaultMask): the part between preTokens and nextTokens is computed; offsets are
      counted from the top-left: visible iff -pre <= j - i <= next. "No mask" is the same
      rule with pre and next at least max(Sq, Skv).
    - 1 (allMask): the full attenMask is given; True (non-zero) means masked. ``mask_rows``
      holds the rows of that mask for the query positions ``i``.
    - 2 (leftUpCausal): lower triangle from the top-left vertex: j <= i.
    - 3 (rightDownCausal): lower triangle from the bottom-right vertex: j <= i + (Skv - Sq).
    - 4 (band, origin at the bottom-right): -pre <= j - i - (Skv - Sq) <= next.
    - 5 / 6 (prefix, uncompressed / compressed): rightDownCausal plus a left rectangle Sq
      high and prefix wide: j <= i + (Skv - Sq) or j < prefix.
    - 7: the band batch uses rule 4, every other batch rule 3.
    - 8: the band batch uses rule 4, every other batch rule 2.
    """
    i = np.asarray(i, dtype=np.int64)
    j = np.asarray(j, dtype=np.int64)
    off = skv - sq
    if sparse_mode == 0:
        rel = j - i
        return (rel >= -pre_tokens) & (rel <= next_tokens)
    if sparse_mode == 1:
        return np.asarray(mask_rows) == 0
    if sparse_mode == 2:
        return j <= i
    if sparse_mode == 3:
        return j <= i + off
    if sparse_mode == 4:
        rel = j - i - off
        return (rel >= -pre_tokens) & (rel <= next_tokens)
    if sparse_mode in (5, 6):
        return (j <= i + off) | (j < prefix_len)
    if sparse_mode == 7:
        if band:
            return visible(4, i, j, sq, skv, pre_tokens=pre_tokens, next_tokens=next_tokens)
        return visible(3, i, j, sq, skv)
    if sparse_mode == 8:
        if band:
            return visible(4, i, j, sq, skv, pre_tokens=pre_tokens, next_tokens=next_tokens)
        return visible(2, i, j, sq, skv)
    raise ValueError(f"unknown sparse_mode {sparse_mode}")


def visible_matrix(sparse_mode: int, sq: int, skv: int, **kw) -> np.ndarray:
    """Full Sq x Skv boolean matrix of visible (i, j) pairs for one batch."""
    i = np.arange(sq)[:, None]
    j = np.arange(skv)[None, :]
    return np.broadcast_to(visible(sparse_mode, i, j, sq, skv, **kw), (sq, skv)).copy()


def count_visible_loops(sparse_mode: int, sq: int, skv: int, *, pre_tokens: int = 0,
                        next_tokens: int = 0, prefix_len: int = 0, band: bool = False,
                        mask=None) -> list:
    """Per-row visible counts by enumerating every (i, j) in plain Python loops.

    Written separately from :func:`visible` (no numpy, one branch per mode) so that the
    vectorised predicate can be checked against it on tiny shapes.
    """
    off = skv - sq
    counts = []
    for i in range(sq):
        n = 0
        for j in range(skv):
            if sparse_mode == 0:
                ok = -pre_tokens <= j - i <= next_tokens
            elif sparse_mode == 1:
                ok = int(mask[i][j]) == 0
            elif sparse_mode == 2 or (sparse_mode == 8 and not band):
                ok = j <= i
            elif sparse_mode == 3 or (sparse_mode == 7 and not band):
                ok = j <= i + off
            elif sparse_mode == 4 or sparse_mode in (7, 8):
                ok = -pre_tokens <= j - i - off <= next_tokens
            elif sparse_mode in (5, 6):
                ok = j <= i + off or j < prefix_len
            else:
                raise ValueError(sparse_mode)
            if ok:
                n += 1
        counts.append(n)
    return counts


# ----------------------------------------------------------------------------------------
# Alibi bias ("压缩mask", section "不同压缩mask的构造方法", alibi scenario: a per-head
# slope times a relative-position bias, in three variants).
# ----------------------------------------------------------------------------------------

ALIBI_MODES = ("right", "sqrt", "left")


def alibi_bias(slope: float, i, j, sq: int, skv: int, mode: str = "right") -> np.ndarray:
    """Alibi bias of query row i and key j (batch-local indices).

    With d = i + (Skv - Sq) - j, the distance from the bottom-right diagonal:
    - "right" (right-aligned bias): slope * (j - i - (Skv - Sq)) = -slope * d;
    - "sqrt" (the right-aligned bias with its magnitude square-rooted):
      -slope * sign(d) * sqrt(|d|);
    - "left" (left-aligned bias, measured from the top-left diagonal): slope * (j - i).
    """
    i = np.asarray(i, dtype=np.float64)
    j = np.asarray(j, dtype=np.float64)
    if mode == "left":
        return float(slope) * (j - i)
    d = i + float(skv - sq) - j
    if mode == "right":
        return -float(slope) * d
    if mode == "sqrt":
        return -float(slope) * np.sign(d) * np.sqrt(np.abs(d))
    raise ValueError(mode)


# ----------------------------------------------------------------------------------------
# The definition, one (batch, head) at a time.
# ----------------------------------------------------------------------------------------

def attention_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, vis: np.ndarray, scale: float,
                   bias: Optional[np.ndarray] = None):
    """O and LSE for one (batch, head): q [R, D], k/v [Skv, D], vis [R, Skv] boolean.

    S = scale * q k^T (+ bias); masked entries are -inf; each row is soft-maxed over its
    visible entries. A row with no visible entry gives O = 0 and LSE = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    rows, d = q.shape
    s = float(scale) * (q @ k.T)
    if bias is not None:
        s = s + bias
    s = np.where(vis, s, -np.inf)
    o = np.zeros((rows, v.shape[1]), dtype=np.float64)
    lse = np.full((rows,), -np.inf, dtype=np.float64)
    live = vis.any(axis=1) if vis.shape[1] else np.zeros(rows, dtype=bool)
    if live.any():
        sl = s[live]
        m = sl.max(axis=1, keepdims=True)
        p = np.exp(sl - m)
        l = p.sum(axis=1, keepdims=True)
        o[live] = (p @ v) / l
        lse[live] = (m + np.log(l))[:, 0]
    return o, lse


def _segments(layout, q, k, sq, skv, actual_seq_qlen, actual_seq_kvlen):
    """Per-batch (q_start, q_len, kv_start, kv_len) and the batch count."""
    if layout == "TND":
        cq = [int(x) for x in actual_seq_qlen]
        ck = [int(x) for x in actual_seq_kvlen]
        # cumulative end offsets, one per batch, no leading zero ("sparseMode介绍",
        # sparseMode=7 example: {3,5} are the lengths 3 and 2).
        qs = [0] + cq[:-1]
        ks = [0] + ck[:-1]
        return [(qs[b], cq[b] - qs[b], ks[b], ck[b] - ks[b]) for b in range(len(cq))]
    nb = q.shape[0]
    return [(0, sq, 0, skv) for _ in range(nb)]


def _head_view(x, layout, b, h, start, length):
    """[length, D] slice of batch b, head h in the given layout."""
    if layout == "BNSD":
        return x[b, h, :length]
    if layout == "BSND":
        return x[b, :length, h]
    return x[start:start + length, h]


def _dims(layout, q, k):
    if layout == "BNSD":
        return q.shape[1], q.shape[2], k.shape[2]
    if layout == "BSND":
        return q.shape[2], q.shape[1], k.shape[1]
    if layout == "TND":
        return q.shape[1], None, None
    raise ValueError(layout)


def _mask_rows(atten_mask, b, h, rows, skv):
    mb = b if atten_mask.shape[0] > 1 else 0
    mh = h if atten_mask.shape[1] > 1 else 0
    return np.asarray(atten_mask[mb, mh])[rows][:, :skv]


def attention(q, k, v, *, layout: str = "BNSD", sparse_mode: int = 0, scale: float,
              pre_tokens: int = 0, next_tokens: int = 0, actual_seq_qlen=None,
              actual_seq_kvlen=None, prefix=None, alibi_slopes=None, atten_mask=None,
              alibi_mode: str = "right"):
    """Full forward pass in fp64. Returns (out, lse).

    Layouts: BNSD q [B, N, Sq, D]; BSND q [B, Sq, N, D]; TND q [T_q, N, D] with the
    cumulative ``actual_seq_qlen`` / ``actual_seq_kvlen``. ``out`` has q's layout; ``lse``
    is [B, N, Sq] (BNSD, BSND) or [N, T_q] (TND). ``atten_mask`` (mode 1) is
    [B or 1, N or 1, Sq, Skv], non-zero = masked. ``prefix`` (modes 5, 6) has one entry per
    batch. ``alibi_slopes`` has one slope per head; ``alibi_mode`` is one of ALIBI_MODES.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, sq, skv = _dims(layout, q, k)
    segs = _segments(layout, q, k, sq, skv, actual_seq_qlen, actual_seq_kvlen)
    band_b = band_batch_index(sparse_mode, [s[1] for s in segs], [s[3] for s in segs])
    out = np.zeros(q.shape[:-1] + (v.shape[-1],), dtype=np.float64)
    if layout == "TND":
        lse = np.full((n, q.shape[0]), -np.inf)
    else:
        lse = np.full((q.shape[0], n, sq), -np.inf)
    for b, (qs, ql, ks, kl) in enumerate(segs):
        pl = int(prefix[b]) if prefix is not None else 0
        for h in range(n):
            rows = np.arange(ql)
            kw = dict(pre_tokens=pre_tokens, next_tokens=next_tokens, prefix_len=pl,
                      band=(b == band_b))
            if sparse_mode == 1:
                kw["mask_rows"] = _mask_rows(atten_mask, b, h, rows, kl)
            vis = np.broadcast_to(
                visible(sparse_mode, rows[:, None], np.arange(kl)[None, :], ql, kl, **kw),
                (ql, kl))
            bias = None
            if alibi_slopes is not None:
                bias = alibi_bias(alibi_slopes[h], rows[:, None], np.arange(kl)[None, :], ql, kl,
                                  alibi_mode)
            qh = _head_view(q, layout, b, h, qs, ql)
            kh = _head_view(k, layout, b, h, ks, kl)
            vh = _head_view(v, layout, b, h, ks, kl)
            o, l = attention_head(qh, kh, vh, vis, scale, bias)
            if layout == "BNSD":
                out[b, h, :ql] = o
                lse[b, h, :ql] = l
            elif layout == "BSND":
                out[b, :ql, h] = o
                lse[b, h, :ql] = l
            else:
                out[qs:qs + ql, h] = o
                lse[h, qs:qs + ql] = l
    return out, lse


def attention_rows(q, k, v, rows: Iterable, *, layout: str = "BNSD", sparse_mode: int = 0,
                   scale: float, pre_tokens: int = 0, next_tokens: int = 0,
                   actual_seq_qlen=None, actual_seq_kvlen=None, prefix=None,
                   alibi_slopes=None, atten_mask=None, alibi_mode: str = "right"):
    """The same definition evaluated only for selected rows ``(b, h, i)`` (i batch-local).

    Used at sizes where a full Sq x Skv matrix per head would take too long. Returns
    (o [R, D], lse [R]) in the order of ``rows``.
    """
    n, sq, skv = _dims(layout, q, k)
    segs = _segments(layout, q, k, sq, skv, actual_seq_qlen, actual_seq_kvlen)
    band_b = band_batch_index(sparse_mode, [s[1] for s in segs], [s[3] for s in segs])
    rows = list(rows)
    o_all = np.zeros((len(rows), v.shape[-1]))
    lse_all = np.zeros((len(rows),))
    for r, (b, h, i) in enumerate(rows):
        qs, ql, ks, kl = segs[b]
        pl = int(prefix[b]) if prefix is not None else 0
        kw = dict(pre_tokens=pre_tokens, next_tokens=next_tokens, prefix_len=pl,
                  band=(b == band_b))
        ii = np.array([i])
        if sparse_mode == 1:
            kw["mask_rows"] = _mask_rows(atten_mask, b, h, ii, kl)
        vis = np.broadcast_to(
            visible(sparse_mode, ii[:, None], np.arange(kl)[None, :], ql, kl, **kw), (1, kl))
        bias = None
        if alibi_slopes is not None:
            bias = alibi_bias(alibi_slopes[h], ii[:, None], np.arange(kl)[None, :], ql, kl,
                              alibi_mode)
        qh = np.asarray(_head_view(q, layout, b, h, qs, ql)[i:i + 1], dtype=np.float64)
        kh = np.asarray(_head_view(k, layout, b, h, ks, kl), dtype=np.float64)
        vh = np.asarray(_head_view(v, layout, b, h, ks, kl), dtype=np.float64)
        o, l = attention_head(qh, kh, vh, vis, scale, bias)
        o_all[r] = o[0]
        lse_all[r] = l[0]
    return o_all, lse_all


# ----------------------------------------------------------------------------------------
# The tiled online-softmax recurrence ("Ý Tưởng Tiling & Online Softmax Trong
# FlashAttention", section "Mục tiêu kiến thức"). A second code path, used only to check
# that the recurrence reaches the definition above.
# ----------------------------------------------------------------------------------------

def tiled_attention(q, k, v, block_size: int, scale: Optional[float] = None, vis=None,
                    bias=None):
    """Block-tiled attention for q [B, Sq, D], k/v [B, Skv, D] with the page's recurrence.

    Rows are processed one Q block at a time; K/V blocks stream past with a running row
    maximum m and running sum l. On each block with maximum m_block:
        m_new = max(m_old, m_block)
        l_new = l_old * exp(m_old - m_new) + sum exp(S_block - m_new)
        O_new = (O_old * l_old * exp(m_old - m_new) + exp(S_block - m_new) V_block) / l_new
    The Sq x Skv matrix is never formed. ``vis`` / ``bias`` ([B, Sq, Skv]) add a mask and a
    bias; rows that have seen only masked entries keep m = -inf, l = 0, O = 0.
    Returns (O [B, Sq, D], LSE [B, Sq]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nb, sq, d = q.shape
    skv = k.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o_out = np.zeros((nb, sq, v.shape[2]))
    lse_out = np.full((nb, sq), -np.inf)
    for b in range(nb):
        for r0 in range(0, sq, block_size):
            r1 = min(r0 + block_size, sq)
            qb = q[b, r0:r1]
            m = np.full((r1 - r0,), -np.inf)
            l = np.zeros((r1 - r0,))
            o = np.zeros((r1 - r0, v.shape[2]))
            for c0 in range(0, skv, block_size):
                c1 = min(c0 + block_size, skv)
                s = scale * (qb @ k[b, c0:c1].T)
                if bias is not None:
                    s = s + bias[b, r0:r1, c0:c1]
                if vis is not None:
                    s = np.where(vis[b, r0:r1, c0:c1], s, -np.inf)
                m_block = s.max(axis=1)
                m_new = np.maximum(m, m_block)
                # Rows with nothing visible yet: keep the shift finite so exp gives 0, not nan.
                shift = np.where(np.isneginf(m_new), 0.0, m_new)
                decay = np.exp(m - shift)
                e = np.exp(s - shift[:, None])
                l_new = l * decay + e.sum(axis=1)
                num = o * (l * decay)[:, None] + e @ v[b, c0:c1]
                safe = np.where(l_new > 0, l_new, 1.0)
                o = np.where((l_new > 0)[:, None], num / safe[:, None], 0.0)
                m, l = m_new, l_new
            o_out[b, r0:r1] = o
            with np.errstate(divide="ignore"):
                lse_out[b, r0:r1] = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return o_out, lse_out
