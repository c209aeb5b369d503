"""GPU parity of the split-KV decode path (at most 16 query rows per sequence) against the fp64
oracle: the decode kernel and its merge of the splits, for every mask mode it takes, the alibi
variants, BNSD / BSND / TND, contiguous and paged K / V, single- and multi-split launches, and
sampled rows of the full-size decode workloads.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from masked_attention_forward_amd import binding as fb
from masked_attention_forward_amd import synth

from test_gpu_parity import DT, _gather, check, make_inputs, run, to64, zero_rows_ok
from test_gpu_paged import run_case

pytestmark = pytest.mark.gpu

DECODE = 3   # fa_plan_stats kernel code of the split-KV decode kernel


def plan(q, k, layout, mode, **kw):
    dims = fb.dims_of(q, k, layout, kw.get("actual_seq_qlen"))
    return fb.fa_plan_stats(dims, layout, mode, **{a: b for a, b in kw.items() if a != "alibi_mode"})


def decode_case(dev, layout, dtype, D, mode, sq, skv, *, B=2, N=3, slopes=None, alibi_mode="right", seed=0,
                **kw):
    q, k, v = make_inputs(layout, dtype, B, N, sq, skv, D, seed=seed)
    st = plan(q, k, layout, mode, **kw)
    assert st["kernel"] == DECODE, st
    o, lse = run(q, k, v, layout, mode, 1.0 / math.sqrt(D), dev, slopes=slopes, alibi_mode=alibi_mode, **kw)
    ref_o, ref_lse = oracle.attention(to64(q), to64(k), to64(v), layout=layout, sparse_mode=mode,
                                      scale=1.0 / math.sqrt(D), alibi_slopes=slopes, alibi_mode=alibi_mode, **kw)
    check(o, lse, ref_o, ref_lse, DT[dtype], f"decode {layout} {dtype} D={D} mode={mode} sq={sq} skv={skv} {kw}")
    zero_rows_ok(o, lse, layout)
    return o, lse


MODE_ARGS = [(0, dict(pre_tokens=300, next_tokens=2)), (0, dict(pre_tokens=5000, next_tokens=-3)), (2, {}),
             (3, {}), (4, dict(pre_tokens=200, next_tokens=0)), (4, dict(pre_tokens=40, next_tokens=9)),
             (5, dict(prefix=[100, 7]))]


@pytest.mark.parametrize("dtype,D,layout", [("bf16", 128, "BNSD"), ("f16", 64, "BSND")])
@pytest.mark.parametrize("sq", [1, 2, 5, 16])
def test_decode_modes(gpu_device, dtype, D, layout, sq):
    """Every mask mode the decode kernel takes, short and long K / V (one split and several:
    the merge), ragged tails, and rows that see nothing (mode 0 with a negative next offset
    empties the first rows)."""
    for mi, (mode, args) in enumerate(MODE_ARGS):
        for skv in (1, 63, 333, 5000):
            if mode == 0 and args.get("next_tokens", 0) < 0 and -args["next_tokens"] >= skv:
                continue
            if mode == 0 and args.get("pre_tokens", 0) < 0 and -args["pre_tokens"] >= sq:
                continue
            decode_case(gpu_device, layout, dtype, D, mode, sq, skv, seed=100 * sq + 10 * mi + skv % 7, **args)


@pytest.mark.parametrize("alibi_mode", ["right", "sqrt", "left"])
def test_decode_alibi(gpu_device, alibi_mode):
    for dtype, D, layout in [("bf16", 128, "BNSD"), ("f16", 64, "BSND")]:
        for sq, skv, mode, args in [(1, 4097, 3, {}), (7, 900, 4, dict(pre_tokens=300, next_tokens=2)),
                                    (16, 2000, 5, dict(prefix=[1000, 3]))]:
            decode_case(gpu_device, layout, dtype, D, mode, sq, skv, slopes=[0.6, 0.25, 0.05],
                        alibi_mode=alibi_mode, seed=300 + sq, **args)


@pytest.mark.parametrize("mode", [3, 5, 7, 8])
def test_decode_tnd(gpu_device, mode):
    """Varlen decode batches: per-sequence query counts 0..16 and key counts 0..6000."""
    ql = [1, 0, 16, 3, 1, 9, 1]
    kl = [6000, 5, 0, 3, 64, 700, 4097]
    if mode == 7:
        kl = [max(a, b) for a, b in zip(ql, kl)]
    band = oracle.band_batch_index(mode, ql, kl)
    kw = {}
    if mode == 7:
        kw = dict(pre_tokens=kl[band], next_tokens=ql[band] - kl[band])
    if mode == 8:
        kw = dict(pre_tokens=kl[band] + 3, next_tokens=ql[band] - kl[band] + 2)
    if mode == 5:
        kw = dict(prefix=[10, 3, 0, 1, 64, 800, 2000])
    for dtype, D in [("bf16", 128), ("f16", 64)]:
        N = 4
        q, k, v = make_inputs("TND", dtype, len(ql), N, 0, 0, D, seed=400 + mode, qlens=ql, kvlens=kl)
        cq, ck = synth.cumulative_ends(ql), synth.cumulative_ends(kl)
        st = plan(q, k, "TND", mode, actual_seq_qlen=cq, actual_seq_kvlen=ck, **kw)
        assert st["kernel"] == DECODE, st
        slopes = synth.alibi_slopes(N) if mode in (3, 5) else None
        o, lse = run(q, k, v, "TND", mode, 0.09, gpu_device, slopes=slopes, actual_seq_qlen=cq,
                     actual_seq_kvlen=ck, **kw)
        ref_o, ref_lse = oracle.attention(to64(q), to64(k), to64(v), layout="TND", sparse_mode=mode, scale=0.09,
                                          actual_seq_qlen=cq, actual_seq_kvlen=ck, alibi_slopes=slopes, **kw)
        check(o, lse, ref_o, ref_lse, DT[dtype], f"decode TND mode={mode} {dtype}")
        zero_rows_ok(o, lse, "TND")


def test_decode_matches_prefill_kernel(gpu_device, monkeypatch):
    q, k, v = make_inputs("BNSD", "bf16", 2, 4, 3, 3000, 128, seed=77)
    o1, l1 = run(q, k, v, "BNSD", 3, 0.0884, gpu_device)
    monkeypatch.setenv("FA_DECODE", "0")
    assert plan(q, k, "BNSD", 3)["kernel"] == 1
    o2, l2 = run(q, k, v, "BNSD", 3, 0.0884, gpu_device)
    ref_o, ref_lse = oracle.attention(to64(q), to64(k), to64(v), layout="BNSD", sparse_mode=3, scale=0.0884)
    check(o1, l1, ref_o, ref_lse, torch.bfloat16, "decode")
    check(o2, l2, ref_o, ref_lse, torch.bfloat16, "prefill kernel")


@pytest.mark.parametrize("cache_layout", ["Norm", "NHSD"])
def test_decode_paged(gpu_device, cache_layout):
    """Decode from paged caches: pages of 64 and 128 keys (decode kernel, bitwise equal to the
    contiguous-K/V decode), 16 keys (generic kernel), TND with empty sequences."""
    for bs in (64, 128, 16):
        for sq, skv, mode, args in [(1, 5000, 3, {}), (4, 700, 4, dict(pre_tokens=300, next_tokens=1)),
                                    (16, 333, 5, dict(prefix=[250, 10]))]:
            run_case(gpu_device, "BNSD", "bf16", 128, mode, bs, cache_layout, sq=sq, skv=skv, seed=500 + sq + bs,
                     **args)
    ql, kl = [1, 0, 16, 2], [3000, 7, 0, 130]
    run_case(gpu_device, "TND", "f16", 64, 3, 64, cache_layout, N=4, qlens=ql, kvlens=kl, seed=555)


def test_decode_empty_and_tiny(gpu_device):
    """No keys at all (every row empty: O = 0, LSE = -inf), one key, and B = 1, N = 1."""
    for B, N, sq, skv in [(2, 3, 1, 0), (1, 1, 1, 1), (1, 1, 16, 1), (3, 1, 2, 64)]:
        q, k, v = make_inputs("BNSD", "bf16", B, N, sq, skv, 128, seed=600 + skv)
        o, lse = run(q, k, v, "BNSD", 3, 0.1, gpu_device)
        ref_o, ref_lse = oracle.attention(to64(q), to64(k), to64(v), layout="BNSD", sparse_mode=3, scale=0.1)
        check(o, lse, ref_o, ref_lse, torch.bfloat16, f"B={B} N={N} sq={sq} skv={skv}")
        zero_rows_ok(o, lse, "BNSD")


def _rows(w, rng, n_random=40):
    rows = []
    if w.layout == "TND":
        for b in range(len(w.qlens)):
            for i in range(w.qlens[b]):
                rows.append((b, int(rng.integers(0, w.N)), i))
        return rows
    for b in {0, w.B - 1}:
        for h in {0, w.N // 2, w.N - 1}:
            for i in range(w.Sq):
                rows.append((b, h, i))
    for _ in range(n_random):
        rows.append((int(rng.integers(0, w.B)), int(rng.integers(0, w.N)), int(rng.integers(0, w.Sq))))
    return rows


@pytest.mark.parametrize("name", ["decode_32k", "decode_spec8_8k", "decode_varlen"])
def test_decode_workloads_sampled_rows(gpu_device, name):
    """The benchmark's decode shapes in the launch configuration bench.py times: sampled rows
    against the oracle, every output finite."""
    w = synth.workloads()[name]
    q, k, v = w.tensors()
    kw = dict(actual_seq_qlen=w.actual_seq_qlen, actual_seq_kvlen=w.actual_seq_kvlen)
    assert plan(q, k, w.layout, w.sparse_mode, **kw)["kernel"] == DECODE
    o, lse = run(q, k, v, w.layout, w.sparse_mode, w.softmax_scale, gpu_device, **kw)
    rows = _rows(w, np.random.default_rng(7))
    qn, kn, vn = (x.float().numpy() for x in (q, k, v))
    ref_o, ref_l = oracle.attention_rows(qn, kn, vn, rows, layout=w.layout, sparse_mode=w.sparse_mode,
                                         scale=w.softmax_scale, **kw)
    got_o, got_l = _gather(o, lse, w, rows)
    check(torch.from_numpy(got_o), torch.from_numpy(got_l), ref_o, ref_l, DT[w.dtype], name)
    assert torch.isfinite(o).all()
    assert torch.isfinite(lse).all()
