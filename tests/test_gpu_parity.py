"""GPU parity: libfa.so (through its C ABI) against the fp64 oracle on the same seeded inputs.

Tolerances (against the fp64 oracle):
  fp32 inputs:       max |dO| <= 1e-5 and max |dLSE| <= 1e-5, both absolute
  fp16 / bf16:       |dO| <= 2e-2 + 1e-2 |O_ref| per element, |dLSE| <= 1e-3
  fully masked rows: O == 0 and LSE == -inf exactly
Mask / visible-pair counts and tile classes are integer work: compared bit-exactly.

The oracle computes on the exact values the GPU sees: the library takes the softmax scale and
the alibi slopes as fp32, so both reach the oracle rounded to fp32 (a slope of 0.6 is
0.60000002384 on the device; over 200 keys that alone moves a bias by 5e-6).

The fp32 LSE bound is absolute. An fp32 number holds an LSE of magnitude X < 256 to within
half an ulp, at most 2^-17 = 7.6e-6; the kernels add the large per-row part of an alibi bias
in double, so what their fp32 arithmetic adds to that rounding is small next to it (an fp32
emulation of the left-aligned band case at |LSE| = 129 gives 7.4e-6 in all). Past 256 half an
ulp alone exceeds 1e-5, so every fp32 case here keeps |LSE| below 256.
"""

import math
import zlib

import numpy as np
import pytest
import torch

import oracle
from masked_attention_forward_amd import binding as fb
from masked_attention_forward_amd import synth

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def to64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def run(q, k, v, layout, mode, scale, dev, slopes=None, mask=None, **kw):
    qd, kd, vd = (x.to(dev).contiguous() for x in (q, k, v))
    sl = torch.tensor(slopes, dtype=torch.float32, device=dev) if slopes is not None else None
    md = torch.from_numpy(np.ascontiguousarray(mask)).to(dev) if mask is not None else None
    print(f"[case] layout={layout} mode={mode} q={tuple(q.shape)} k={tuple(k.shape)} dtype={q.dtype} "
          f"alibi={slopes is not None} kw={ {a: b for a, b in kw.items() if not isinstance(b, list) or len(b) < 20} }",
          flush=True)
    o, lse = fb.flash_attention(qd, kd, vd, layout=layout, sparse_mode=mode, scale=scale,
                                alibi_slopes=sl, atten_mask=md, **kw)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def check(o, lse, ref_o, ref_lse, dtype, what=""):
    o = to64(o)
    lse = lse.double().numpy()
    empty = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: empty-row pattern differs"
    live = ~empty
    if dtype == torch.float32:
        err = np.abs(o - ref_o)
        assert err.max(initial=0) <= 1e-5, f"{what}: max |dO| {err.max()}"
        lse_err = np.abs(lse[live] - ref_lse[live])
        assert np.abs(ref_lse[live]).max(initial=0) < 256, f"{what}: |LSE| past the range of the bound"
        assert lse_err.max(initial=0) <= 1e-5, f"{what}: max |dLSE| {lse_err.max(initial=0)}"
    else:
        bound = 2e-2 + 1e-2 * np.abs(ref_o)
        bad = np.abs(o - ref_o) > bound
        assert not bad.any(), f"{what}: {bad.sum()} elements out of tolerance, max err {np.abs(o - ref_o).max()}"
        assert np.abs(lse[live] - ref_lse[live]).max(initial=0) <= 1e-3, \
            f"{what}: max |dLSE| {np.abs(lse[live] - ref_lse[live]).max()}"


def f32_exact(x):
    """x as the fp32 value the library receives (scale, alibi slopes)."""
    if x is None:
        return None
    if isinstance(x, (list, tuple, np.ndarray)):
        return [float(np.float32(v)) for v in x]
    return float(np.float32(x))


def ref_attention(q, k, v, *, scale, alibi_slopes=None, **kw):
    """The oracle on the exact inputs the GPU sees (fp32 scale and slopes)."""
    return oracle.attention(q, k, v, scale=f32_exact(scale), alibi_slopes=f32_exact(alibi_slopes), **kw)


def zero_rows_ok(o, lse, layout):
    """O rows whose LSE is -inf must be exactly zero."""
    o = to64(o)
    lse = lse.numpy()
    if layout == "BNSD":
        rows = o[np.isneginf(lse)]
    elif layout == "BSND":
        rows = o.transpose(0, 2, 1, 3)[np.isneginf(lse)]
    else:
        rows = o.transpose(1, 0, 2)[np.isneginf(lse)]
    assert np.all(rows == 0.0)


def make_inputs(layout, dtype, B, N, sq, skv, D, seed, qlens=None, kvlens=None):
    w = synth.Workload("t", layout, dtype, B, N, D, sq, skv, qlens=qlens, kvlens=kvlens, seed=seed)
    return w.tensors()


# ---------------------------------------------------------------------------------------
# Mask probe: device mask code vs the oracle's predicate, bit-exact.
# ---------------------------------------------------------------------------------------

def brute_class(vis, bm, bn, n_kv_max):
    sq, skv = vis.shape
    rows = []
    for i0 in range(0, sq, bm):
        r = []
        for kt in range(n_kv_max):
            j0 = kt * bn
            if j0 >= skv:
                r.append(3)
                continue
            blk = vis[i0:i0 + bm, j0:j0 + bn]
            if not blk.any():
                r.append(0)
            elif j0 + bn <= skv and blk.all():
                r.append(2)
            else:
                r.append(1)
        rows.append(r)
    return rows


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 16)])
@pytest.mark.parametrize("mode", [0, 2, 3, 4, 5, 6])
def test_probe_exact_bnsd(gpu_device, dtype, D, mode):
    rng = np.random.default_rng(900 + mode)
    for _ in range(6):
        sq, skv = int(rng.integers(0, 400)), int(rng.integers(0, 400))
        while True:
            pre = int(rng.integers(-sq, sq + skv + 3))
            nxt = int(rng.integers(-skv, sq + skv + 3))
            if mode == 0 and ((nxt < 0 and not (pre >= -nxt and -nxt < max(skv, 1))) or
                              (pre < 0 and not (nxt >= -pre and -pre < max(sq, 1)))):
                continue
            if mode == 4 and pre + nxt < 0:
                continue
            break
        B, N = 2, 2
        prefix = [int(rng.integers(0, skv + 2)) for _ in range(B)]
        dims = fb.make_dims(DT[dtype], 0, B=B, N=N, Sq=sq, Skv=skv, D=D)
        print(f"[probe] mode={mode} sq={sq} skv={skv} pre={pre} next={nxt} prefix={prefix}", flush=True)
        counts, tiles = fb.fa_mask_probe(dims, "BNSD", mode, device=gpu_device, pre_tokens=pre,
                                         next_tokens=nxt, prefix=prefix)
        torch.cuda.synchronize()
        counts = counts.cpu().numpy()
        bm, bn, nq, nk = fb.fa_tile_shape(dims, "BNSD")
        exp_tiles = []
        for b in range(B):
            vis = oracle.visible_matrix(mode, sq, skv, pre_tokens=pre, next_tokens=nxt, prefix_len=prefix[b])
            for h in range(N):
                assert counts[b, h].tolist() == vis.sum(axis=1).tolist()
            exp_tiles += brute_class(vis, bm, bn, nk)
        if nq and nk:
            assert tiles.cpu().numpy().tolist() == exp_tiles


@pytest.mark.parametrize("mode", [3, 7, 8])
def test_probe_exact_tnd(gpu_device, mode):
    rng = np.random.default_rng(950 + mode)
    for _ in range(6):
        nb = int(rng.integers(1, 6))
        ql = [int(x) for x in rng.integers(0, 300, nb)]
        kl = [int(x) for x in rng.integers(0, 300, nb)]
        if mode == 7:
            kl = [max(a, b) for a, b in zip(ql, kl)]
        band = oracle.band_batch_index(mode, ql, kl)
        pre = nxt = 0
        if band is not None:
            pre = kl[band] + int(rng.integers(0, 4))
            nxt = int(rng.integers(ql[band] - kl[band], 1)) if mode == 7 else ql[band] - kl[band] + int(rng.integers(0, 4))
        cq, ck = synth.cumulative_ends(ql), synth.cumulative_ends(kl)
        dims = fb.make_dims(torch.bfloat16, 2, B=nb, N=2, D=128, T_q=sum(ql), T_kv=sum(kl))
        print(f"[probe-tnd] mode={mode} ql={ql} kl={kl} pre={pre} next={nxt}", flush=True)
        counts, tiles = fb.fa_mask_probe(dims, "TND", mode, device=gpu_device, pre_tokens=pre, next_tokens=nxt,
                                         actual_seq_qlen=cq, actual_seq_kvlen=ck)
        torch.cuda.synchronize()
        counts = counts.cpu().numpy()
        bm, bn, nq, nk = fb.fa_tile_shape(dims, "TND", cq, ck)
        exp_tiles = []
        start = 0
        for b in range(nb):
            vis = oracle.visible_matrix(mode, ql[b], kl[b], pre_tokens=pre, next_tokens=nxt, band=(b == band))
            for h in range(2):
                assert counts[h, start:start + ql[b]].tolist() == vis.sum(axis=1).tolist()
            exp_tiles += brute_class(vis, bm, bn, nk)
            start += ql[b]
        if nq and nk:
            assert tiles.cpu().numpy().tolist() == exp_tiles


def test_probe_dense_mask_counts(gpu_device):
    rng = np.random.default_rng(77)
    B, N, sq, skv = 2, 3, 70, 133
    for bc in ([0, 0], [1, 0], [0, 1], [1, 1]):
        mb, mh = (1 if bc[0] else B), (1 if bc[1] else N)
        mask = (rng.random((mb, mh, sq, skv)) < 0.6).astype(np.uint8)
        dims = fb.make_dims(torch.bfloat16, 0, B=B, N=N, Sq=sq, Skv=skv, D=128)
        counts, _ = fb.fa_mask_probe(dims, "BNSD", 1, device=gpu_device,
                                     atten_mask=torch.from_numpy(mask).to(gpu_device), mask_bcast=bc)
        counts = counts.cpu().numpy()
        for b in range(B):
            for h in range(N):
                m = mask[0 if bc[0] else b, 0 if bc[1] else h]
                assert counts[b, h].tolist() == (m == 0).sum(axis=1).tolist()


# ---------------------------------------------------------------------------------------
# Small-shape parity over modes, dtypes, layouts, head sizes (several tiles + ragged tails)
# ---------------------------------------------------------------------------------------

VARIANTS = [("bf16", 128, "BNSD"), ("f16", 128, "BSND"), ("bf16", 64, "BSND"), ("f16", 64, "BNSD"),
            ("f32", 16, "BNSD"), ("f32", 128, "BSND"), ("bf16", 40, "BNSD")]

MODE_ARGS = {
    0: [dict(pre_tokens=synth.NO_MASK, next_tokens=synth.NO_MASK), dict(pre_tokens=9, next_tokens=-3),
        dict(pre_tokens=-3, next_tokens=70), dict(pre_tokens=100, next_tokens=0), dict(pre_tokens=5, next_tokens=20)],
    2: [{}], 3: [{}], 4: [dict(pre_tokens=60, next_tokens=0), dict(pre_tokens=30, next_tokens=-10)],
    5: [dict(prefix=[0, 150])], 6: [dict(prefix=[77, 3])],
}


@pytest.mark.parametrize("mode", [0, 2, 3, 4, 5, 6])
@pytest.mark.parametrize("alibi", [False, True])
def test_parity_small(gpu_device, mode, alibi):
    for vi, (dtype, D, layout) in enumerate(VARIANTS):
        for (sq, skv) in [(300, 200), (130, 333)]:
            for args in MODE_ARGS[mode]:
                B, N = 2, 3
                q, k, v = make_inputs(layout, dtype, B, N, sq, skv, D, seed=1000 * mode + 10 * vi + sq % 7)
                if mode == 0 and args.get("next_tokens", 0) < 0 and -args["next_tokens"] >= skv:
                    continue
                if mode == 0 and args.get("pre_tokens", 0) < 0 and -args["pre_tokens"] >= sq:
                    continue
                slopes = synth.alibi_slopes(N) if alibi else None
                scale = 1.0 / math.sqrt(D)
                o, lse = run(q, k, v, layout, mode, scale, gpu_device, slopes=slopes, **args)
                ref_o, ref_lse = ref_attention(to64(q), to64(k), to64(v), layout=layout, sparse_mode=mode,
                                                  scale=scale, alibi_slopes=slopes, **args)
                check(o, lse, ref_o, ref_lse, DT[dtype], f"mode={mode} {dtype} D={D} {layout} {sq}x{skv} {args}")
                zero_rows_ok(o, lse, layout)


@pytest.mark.parametrize("alibi", [False, True])
def test_parity_dense_mask(gpu_device, alibi):
    rng = np.random.default_rng(31)
    for dtype, D, layout in VARIANTS[:5]:
        B, N, sq, skv = 2, 3, 150, 170
        q, k, v = make_inputs(layout, dtype, B, N, sq, skv, D, seed=55)
        for bc in ([0, 0], [1, 1], [1, 0]):
            mb, mh = (1 if bc[0] else B), (1 if bc[1] else N)
            mask = (rng.random((mb, mh, sq, skv)) < 0.7).astype(np.uint8)
            mask[..., 5, :] = 1     # a fully masked row
            slopes = synth.alibi_slopes(N) if alibi else None
            o, lse = run(q, k, v, layout, 1, 0.1, gpu_device, slopes=slopes, mask=mask, mask_bcast=bc)
            ref_o, ref_lse = ref_attention(to64(q), to64(k), to64(v), layout=layout, sparse_mode=1, scale=0.1,
                                              atten_mask=mask, alibi_slopes=slopes)
            check(o, lse, ref_o, ref_lse, DT[dtype], f"mode=1 {dtype} {layout} bcast={bc}")
            zero_rows_ok(o, lse, layout)


ALIBI_VARIANTS = [("bf16", 128, "BNSD"), ("f16", 64, "BSND"), ("f32", 16, "BNSD"), ("bf16", 40, "BSND")]
ALIBI_CASES = [(0, dict(pre_tokens=40, next_tokens=25)), (3, {}), (4, dict(pre_tokens=60, next_tokens=7)),
               (5, dict(prefix=[250, 10]))]
ALIBI_SLOPES = [0.6, 0.25, 0.05]


@pytest.mark.parametrize("alibi_mode", ["sqrt", "left"])
def test_parity_alibi_variants(gpu_device, alibi_mode):
    """Square-root and left-aligned alibi ("压缩mask", alibi scenario) against the oracle: the
    MFMA kernel (D 128 and 64) and the generic kernel; masks with keys on both sides of the
    bottom-right diagonal, a prefix, and varlen TND (per-batch diagonal shift)."""
    for vi, (dtype, D, layout) in enumerate(ALIBI_VARIANTS):
        for mode, args in ALIBI_CASES:
            for (sq, skv) in [(300, 200), (130, 333)]:
                B, N = 2, 3
                q, k, v = make_inputs(layout, dtype, B, N, sq, skv, D, seed=7000 + 10 * vi + mode)
                scale = 1.0 / math.sqrt(D)
                o, lse = run(q, k, v, layout, mode, scale, gpu_device, slopes=ALIBI_SLOPES,
                             alibi_mode=alibi_mode, **args)
                ref_o, ref_lse = ref_attention(to64(q), to64(k), to64(v), layout=layout, sparse_mode=mode,
                                                  scale=scale, alibi_slopes=ALIBI_SLOPES, alibi_mode=alibi_mode,
                                                  **args)
                check(o, lse, ref_o, ref_lse, DT[dtype],
                      f"alibi={alibi_mode} mode={mode} {dtype} D={D} {layout} {sq}x{skv} {args}")
                zero_rows_ok(o, lse, layout)
    ql, kl = [200, 1, 129, 257], [150, 300, 64, 257]
    for dtype, D in [("bf16", 128), ("f32", 32)]:
        q, k, v = make_inputs("TND", dtype, len(ql), 3, 0, 0, D, seed=7100, qlens=ql, kvlens=kl)
        cq, ck = synth.cumulative_ends(ql), synth.cumulative_ends(kl)
        o, lse = run(q, k, v, "TND", 3, 0.125, gpu_device, slopes=ALIBI_SLOPES, alibi_mode=alibi_mode,
                     actual_seq_qlen=cq, actual_seq_kvlen=ck)
        ref_o, ref_lse = ref_attention(to64(q), to64(k), to64(v), layout="TND", sparse_mode=3, scale=0.125,
                                          actual_seq_qlen=cq, actual_seq_kvlen=ck, alibi_slopes=ALIBI_SLOPES,
                                          alibi_mode=alibi_mode)
        check(o, lse, ref_o, ref_lse, DT[dtype], f"alibi={alibi_mode} TND {dtype}")


@pytest.mark.parametrize("alibi_mode", [None, "right", "sqrt", "left"])
def test_parity_mfma32_kernel(gpu_device, alibi_mode, monkeypatch):
    """The 4-wave MFMA kernel (FA_KERNEL=mfma32, kept for comparisons) against the oracle."""
    monkeypatch.setenv("FA_KERNEL", "mfma32")
    dims = fb.make_dims(torch.bfloat16, 0, B=1, N=1, Sq=64, Skv=64, D=128)   # > 16 rows: not decode
    assert fb.fa_tile_shape(dims, "BNSD")[:2] == (128, 64)
    slopes = ALIBI_SLOPES if alibi_mode else None
    for dtype, D, layout in [("bf16", 128, "BNSD"), ("f16", 64, "BSND")]:
        for mode, args in [(0, dict(pre_tokens=9, next_tokens=-3))] + ALIBI_CASES[1:]:
            q, k, v = make_inputs(layout, dtype, 2, 3, 300, 333, D, seed=7200 + mode)
            kw = dict(alibi_mode=alibi_mode) if alibi_mode else {}
            o, lse = run(q, k, v, layout, mode, 0.1, gpu_device, slopes=slopes, **kw, **args)
            ref_o, ref_lse = ref_attention(to64(q), to64(k), to64(v), layout=layout, sparse_mode=mode,
                                              scale=0.1, alibi_slopes=slopes, alibi_mode=alibi_mode or "right",
                                              **args)
            check(o, lse, ref_o, ref_lse, DT[dtype], f"mfma32 alibi={alibi_mode} mode={mode} {dtype} {layout}")
            zero_rows_ok(o, lse, layout)


@pytest.mark.parametrize("mode", [3, 5, 7, 8])
@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f16", 64), ("f32", 32)])
def test_parity_tnd(gpu_device, mode, dtype, D):
    rng = np.random.default_rng(4000 + mode)
    ql = [200, 0, 1, 129, 64, 257]
    kl = [150, 5, 0, 300, 64, 257]
    if mode == 7:
        kl = [max(a, b) for a, b in zip(ql, kl)]
    band = oracle.band_batch_index(mode, ql, kl)
    kw = {}
    if mode == 7:
        kw = dict(pre_tokens=kl[band], next_tokens=ql[band] - kl[band])
    if mode == 8:
        kw = dict(pre_tokens=kl[band] + 3, next_tokens=ql[band] - kl[band] + 2)
    if mode == 5:
        kw = dict(prefix=[int(x) for x in rng.integers(0, 320, len(ql))])
    N = 4
    q, k, v = make_inputs("TND", dtype, len(ql), N, 0, 0, D, seed=77 + mode, qlens=ql, kvlens=kl)
    cq, ck = synth.cumulative_ends(ql), synth.cumulative_ends(kl)
    slopes = synth.alibi_slopes(N) if mode in (3, 5) else None
    o, lse = run(q, k, v, "TND", mode, 0.09, gpu_device, slopes=slopes, actual_seq_qlen=cq, actual_seq_kvlen=ck, **kw)
    ref_o, ref_lse = ref_attention(to64(q), to64(k), to64(v), layout="TND", sparse_mode=mode, scale=0.09,
                                      actual_seq_qlen=cq, actual_seq_kvlen=ck, alibi_slopes=slopes, **kw)
    check(o, lse, ref_o, ref_lse, DT[dtype], f"TND mode={mode} {dtype}")
    zero_rows_ok(o, lse, "TND")


@pytest.mark.parametrize("name", ["tiny_f32", "tiny_f32_causal"])
def test_page_example_tiny_f32(gpu_device, name):
    """Exercise page example 1 (seed 42, (2,12,16)) as fp32 BNSD with one head: no mask and
    the causal variant pre=12, next=0; max |dO| <= 1e-5 against the fp64 oracle."""
    w = synth.workloads()[name]
    q, k, v = w.tensors()
    o, lse = run(q, k, v, "BNSD", w.sparse_mode, w.softmax_scale, gpu_device, pre_tokens=w.pre_tokens,
                 next_tokens=w.next_tokens)
    ref_o, ref_lse = ref_attention(to64(q), to64(k), to64(v), layout="BNSD", sparse_mode=w.sparse_mode,
                                      scale=w.softmax_scale, pre_tokens=w.pre_tokens, next_tokens=w.next_tokens)
    check(o, lse, ref_o, ref_lse, torch.float32, name)


def test_band_negative_next_16(gpu_device):
    """sparseMode=0, preTokens=9, nextTokens=-3 at Sq=Skv=16, D=128 bf16: full comparison,
    rows 0-2 fully masked."""
    w = synth.workloads()["band_neg_16"]
    q, k, v = w.tensors()
    o, lse = run(q, k, v, "BNSD", 0, w.softmax_scale, gpu_device, pre_tokens=9, next_tokens=-3)
    ref_o, ref_lse = ref_attention(to64(q), to64(k), to64(v), layout="BNSD", sparse_mode=0,
                                      scale=w.softmax_scale, pre_tokens=9, next_tokens=-3)
    check(o, lse, ref_o, ref_lse, torch.bfloat16, "band_neg_16")
    assert np.all(np.isneginf(lse.numpy()[0, 0, :3]))
    assert np.all(to64(o)[0, 0, :3] == 0)


# ---------------------------------------------------------------------------------------
# Query split (sparseMode 7 / 8) reproduces the unsplit rows
# ---------------------------------------------------------------------------------------

def _split_compare(dev, unsplit, shards, N, D, dtype, seed):
    """unsplit = (mode, qlens, kvlens, kw); shards = [(mode, [(ub, r0, n)], kw)]."""
    mode_u, qlens, kvlens, kw_u = unsplit
    g = torch.Generator().manual_seed(seed)
    qs = [torch.randn(n, N, D, generator=g).to(DT[dtype]) for n in qlens]
    ks = [torch.randn(n, N, D, generator=g).to(DT[dtype]) for n in kvlens]
    vs = [torch.randn(n, N, D, generator=g).to(DT[dtype]) for n in kvlens]
    cq, ck = synth.cumulative_ends(qlens), synth.cumulative_ends(kvlens)
    o_u, l_u = run(torch.cat(qs), torch.cat(ks), torch.cat(vs), "TND", mode_u, 0.088, dev,
                   actual_seq_qlen=cq, actual_seq_kvlen=ck, **kw_u)
    starts = [0] + cq[:-1]
    for mode_s, parts, kw in shards:
        q = torch.cat([qs[ub][r0:r0 + n] for ub, r0, n in parts])
        k = torch.cat([ks[ub] for ub, _, _ in parts])
        v = torch.cat([vs[ub] for ub, _, _ in parts])
        sq = synth.cumulative_ends([n for _, _, n in parts])
        sk = synth.cumulative_ends([kvlens[ub] for ub, _, _ in parts])
        o_s, l_s = run(q, k, v, "TND", mode_s, 0.088, dev, actual_seq_qlen=sq, actual_seq_kvlen=sk, **kw)
        row = 0
        for ub, r0, n in parts:
            src = starts[ub] + r0
            assert torch.equal(o_s[row:row + n], o_u[src:src + n]), (mode_s, ub, r0, n)
            assert torch.equal(l_s[:, row:row + n], l_u[:, src:src + n]), (mode_s, ub, r0, n)
            row += n


def test_split_page_examples_gpu(gpu_device):
    """The sparseMode=7 and =8 worked examples on the GPU: shards == unsplit, bitwise."""
    _split_compare(gpu_device, (3, [3, 4, 5, 4], [3, 6, 5, 4], {}),
                   [(7, [(0, 0, 3), (1, 0, 2)], dict(pre_tokens=6, next_tokens=-2)),
                    (3, [(1, 2, 2), (2, 0, 5), (3, 0, 4)], {})], N=2, D=128, dtype="bf16", seed=7)
    _split_compare(gpu_device, (2, [3, 5, 5, 4], [3, 4, 5, 4], {}),
                   [(2, [(0, 0, 3), (1, 0, 2)], {}),
                    (8, [(1, 2, 3), (2, 0, 5), (3, 0, 4)], dict(pre_tokens=4, next_tokens=1))],
                   N=2, D=128, dtype="bf16", seed=8)


def test_split_varlen_config(gpu_device):
    """Varlen TND config (16 lengths U[128, 4096], N=32, D=128, bf16): the last sequence's
    queries cut in two (mode 7 band shard + mode 3 shard) give the unsplit mode-3 rows; the
    mirror cut of the first sequence (mode 2 shard + mode 8 band shard) gives the unsplit
    mode-2 rows."""
    w = synth.workloads()["varlen_tnd"]
    L = w.qlens
    last = len(L) - 1
    q1 = L[last] // 2
    shard_a = [(b, 0, L[b]) for b in range(last)] + [(last, 0, q1)]
    _split_compare(gpu_device, (3, L, L, {}),
                   [(7, shard_a, dict(pre_tokens=L[last], next_tokens=q1 - L[last])),
                    (3, [(last, q1, L[last] - q1)], {})], N=32, D=128, dtype="bf16", seed=4)
    q0 = L[0] // 2
    shard_2 = [(0, q0, L[0] - q0)] + [(b, 0, L[b]) for b in range(1, len(L))]
    _split_compare(gpu_device, (2, L, L, {}),
                   [(2, [(0, 0, q0)], {}),
                    (8, shard_2, dict(pre_tokens=L[0], next_tokens=0))],
                   N=32, D=128, dtype="bf16", seed=5)


# ---------------------------------------------------------------------------------------
# Full-size configs: sampled rows against the oracle
# ---------------------------------------------------------------------------------------

def _sample_rows(w, rng, n_random=24):
    rows = []
    if w.layout == "TND":
        bs = [0, len(w.qlens) // 2, len(w.qlens) - 1]
        for b in bs:
            L = w.qlens[b]
            for h in (0, w.N - 1):
                for i in {0, 1, min(127, L - 1), min(128, L - 1), L // 2, L - 1}:
                    rows.append((b, h, i))
        for _ in range(n_random):
            b = int(rng.integers(0, len(w.qlens)))
            rows.append((b, int(rng.integers(0, w.N)), int(rng.integers(0, w.qlens[b]))))
        return rows
    for b in {0, w.B - 1}:
        for h in {0, w.N // 2, w.N - 1}:
            for i in {0, 1, 127, 128, 255, 256, 257, w.Sq // 2, w.Sq - 2, w.Sq - 1}:
                rows.append((b, h, i))
    for _ in range(n_random):
        rows.append((int(rng.integers(0, w.B)), int(rng.integers(0, w.N)), int(rng.integers(0, w.Sq))))
    return rows


def _gather(o, lse, w, rows):
    o = to64(o) if not isinstance(o, np.ndarray) else o
    lse = lse.double().numpy()
    out_o, out_l = [], []
    starts = [0] + (w.actual_seq_qlen[:-1] if w.layout == "TND" else [])
    for b, h, i in rows:
        if w.layout == "BNSD":
            out_o.append(o[b, h, i]); out_l.append(lse[b, h, i])
        elif w.layout == "BSND":
            out_o.append(o[b, i, h]); out_l.append(lse[b, h, i])
        else:
            out_o.append(o[starts[b] + i, h]); out_l.append(lse[h, starts[b] + i])
    return np.array(out_o), np.array(out_l)


def _whole_slices(w):
    """(batch, head) slices compared element by element at full size: every slice of the
    headline, else 8 slices whose heads cover every residue mod 8. Work items of one (batch,
    head) run on the XCD its index selects modulo 8 (heads are the fastest index), so this
    covers the work of every XCD."""
    nb = len(w.qlens) if w.layout == "TND" else w.B
    if w.name == "causal_8192":
        return [(b, h) for b in range(nb) for h in range(w.N)]
    return [((r * nb) // 8, (5 * r) % w.N) for r in range(8)]


def _slice_problem(w, q, k, v, b, h):
    """q, k, v of slice (b, h) as a one-batch, one-head problem in the workload's layout, and
    the oracle keyword arguments that go with it."""
    kw = dict(layout=w.layout, sparse_mode=w.sparse_mode, scale=w.softmax_scale, pre_tokens=w.pre_tokens,
              next_tokens=w.next_tokens, alibi_slopes=[w.slopes()[h]] if w.alibi else None,
              prefix=[w.prefix[b]] if w.prefix is not None else None)
    if w.layout == "BNSD":
        return q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1], kw
    if w.layout == "BSND":
        return q[b:b + 1, :, h:h + 1], k[b:b + 1, :, h:h + 1], v[b:b + 1, :, h:h + 1], kw
    assert w.sparse_mode not in (7, 8), "a one-sequence slice would move the band batch"
    qe, ke = w.actual_seq_qlen, w.actual_seq_kvlen
    qs, ks = (qe[b - 1] if b else 0), (ke[b - 1] if b else 0)
    kw.update(actual_seq_qlen=[qe[b] - qs], actual_seq_kvlen=[ke[b] - ks])
    return q[qs:qe[b], h:h + 1], k[ks:ke[b], h:h + 1], v[ks:ke[b], h:h + 1], kw


def _slice_of(o, lse, w, b, h):
    """The GPU's O [rows, D] and LSE [rows] of slice (b, h)."""
    if w.layout == "BNSD":
        return o[b, h], lse[b, h]
    if w.layout == "BSND":
        return o[b, :, h], lse[b, h]
    qe = w.actual_seq_qlen
    qs = qe[b - 1] if b else 0
    return o[qs:qe[b], h], lse[h, qs:qe[b]]


@pytest.mark.parametrize("name", ["causal_2048", "band_8192", "band_neg_8192", "causal_8192",
                                  "varlen_tnd", "prefix_alibi", "prefix_alibi_square", "causal_8192_mask"])
def test_config_full_size(gpu_device, name):
    """Each full-size workload, run once in the launch configuration bench.py times, against
    the oracle: whole (batch, head) slices element by element (all 64 of the headline, 8 of
    every other workload), plus sampled rows at tile boundaries of other slices."""
    w = synth.workloads()[name]
    q, k, v = w.tensors()
    kw = dict(pre_tokens=w.pre_tokens, next_tokens=w.next_tokens, prefix=w.prefix,
              actual_seq_qlen=w.actual_seq_qlen, actual_seq_kvlen=w.actual_seq_kvlen)
    mask, bcast = w.mask()
    o, lse = run(q, k, v, w.layout, w.sparse_mode, w.softmax_scale, gpu_device, slopes=w.slopes(),
                 mask=None if mask is None else mask.numpy(), mask_bcast=bcast, **kw)
    assert torch.isfinite(o).all()
    assert not torch.isnan(lse).any()
    qn, kn, vn = (x.float().numpy() for x in (q, k, v))
    on, ln = o.float().numpy(), lse.numpy()
    slices = _whole_slices(w)
    print(f"[full] {name}: {len(slices)} whole slices", flush=True)
    for b, h in slices:
        qs, ks, vs, okw = _slice_problem(w, qn, kn, vn, b, h)
        if mask is not None:
            okw["atten_mask"] = mask.numpy()   # [1, 1, Sq, Skv]: the same for every slice
        ref_o, ref_l = ref_attention(qs.astype(np.float64), ks.astype(np.float64), vs.astype(np.float64), **okw)
        got_o, got_l = _slice_of(on, ln, w, b, h)
        ref_o = ref_o.reshape(got_o.shape)
        ref_l = ref_l.reshape(got_l.shape)
        check(torch.from_numpy(got_o), torch.from_numpy(got_l), ref_o, ref_l, DT[w.dtype], f"{name} slice ({b}, {h})")
    # Sampled rows of the remaining slices (tile edges and random rows; a stable seed).
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    rows = _sample_rows(w, rng)
    ref_o, ref_l = oracle.attention_rows(qn, kn, vn, rows, layout=w.layout, sparse_mode=w.sparse_mode,
                                         scale=f32_exact(w.softmax_scale), alibi_slopes=f32_exact(w.slopes()),
                                         atten_mask=None if mask is None else mask.numpy(), **kw)
    got_o, got_l = _gather(o, lse, w, rows)
    check(torch.from_numpy(got_o), torch.from_numpy(got_l), ref_o, ref_l, DT[w.dtype], f"{name} sampled rows")


@pytest.mark.parametrize("layout", ["TND", "BNSD"])
def test_table_order_does_not_change_results(gpu_device, monkeypatch, layout):
    """The table launch order (sequence-major or longest first) only decides which workgroup
    runs an item when; every item's arithmetic is the same, so the outputs are bitwise equal.
    The sequence-major run is also checked against the oracle."""
    if layout == "TND":
        ql = [300, 5, 129, 0, 640, 64, 200]
        kl = [300, 9, 200, 3, 640, 64, 333]
        q, k, v = make_inputs("TND", "bf16", len(ql), 8, 0, 0, 128, seed=91, qlens=ql, kvlens=kl)
        kw = dict(actual_seq_qlen=synth.cumulative_ends(ql), actual_seq_kvlen=synth.cumulative_ends(kl))
        mode = 3
    else:
        q, k, v = make_inputs("BNSD", "bf16", 3, 8, 300, 520, 128, seed=92)
        kw = dict(prefix=[0, 77, 400])
        mode = 5
    res = {}
    for order in ("seq", "lpt"):
        monkeypatch.setenv("FA_TABLE_ORDER", order)
        res[order] = run(q, k, v, layout, mode, 0.088, gpu_device, **kw)
    assert torch.equal(res["seq"][0], res["lpt"][0]) and torch.equal(res["seq"][1], res["lpt"][1])
    ref_o, ref_lse = ref_attention(to64(q), to64(k), to64(v), layout=layout, sparse_mode=mode, scale=0.088, **kw)
    check(res["seq"][0], res["seq"][1], ref_o, ref_lse, DT["bf16"], f"table order {layout}")


def test_deterministic(gpu_device):
    w = synth.workloads()["causal_2048"]
    q, k, v = w.tensors()
    a = run(q, k, v, "BNSD", 3, w.softmax_scale, gpu_device)
    b = run(q, k, v, "BNSD", 3, w.softmax_scale, gpu_device)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# ---------------------------------------------------------------------------------------
# Empty and degenerate inputs
# ---------------------------------------------------------------------------------------

def test_empty_inputs(gpu_device):
    dev = gpu_device
    for dtype in ("bf16", "f32"):
        for (B, sq, skv) in [(0, 5, 5), (2, 0, 7), (2, 7, 0), (1, 1, 1)]:
            q, k, v = make_inputs("BNSD", dtype, B, 2, sq, skv, 128, seed=3)
            o, lse = run(q, k, v, "BNSD", 3 if skv >= sq else 2, 0.1, dev)
            ref_o, ref_lse = ref_attention(to64(q), to64(k), to64(v), layout="BNSD",
                                              sparse_mode=3 if skv >= sq else 2, scale=0.1)
            assert o.shape == q.shape and lse.shape == (B, 2, sq)
            if o.numel():
                check(o, lse, ref_o, ref_lse, DT[dtype], f"empty {B} {sq} {skv}")
    # TND with zero-length sequences and an empty total
    q, k, v = make_inputs("TND", "bf16", 3, 2, 0, 0, 128, seed=4, qlens=[0, 0, 0], kvlens=[0, 4, 0])
    o, lse = run(q, k, v, "TND", 3, 0.1, dev, actual_seq_qlen=[0, 0, 0], actual_seq_kvlen=[0, 4, 4])
    assert o.numel() == 0 and lse.shape == (2, 0)


def test_single_key_rows_return_value(gpu_device):
    """sparseMode=0 with pre=next=0 leaves only the diagonal: O_i = v_i (to bf16 rounding of
    P = 1, exact) and LSE_i = scale q_i.k_i."""
    q, k, v = make_inputs("BNSD", "bf16", 1, 2, 200, 200, 128, seed=9)
    o, lse = run(q, k, v, "BNSD", 0, 0.1, gpu_device, pre_tokens=0, next_tokens=0)
    assert torch.equal(o, v)
    ref = 0.1 * (to64(q) * to64(k)).sum(-1)
    assert np.abs(lse.double().numpy() - ref).max() < 1e-4


@pytest.mark.parametrize("mode", [0, 3])
def test_softmax_row_max_growth(gpu_device, mode):
    """Row maxima that move after the first tile. The kernel exponentiates each tile against
    the row maximum it already holds and switches to the exact update (tile maximum, rescale)
    only when a lane's sum of a tile's 32 values exceeds 2^15 or overflows. Head 0: scores
    climb about 20 (log2 units) per 64-key tile, so every tile needs the exact update; head 1:
    about 6 per tile, so the held maximum goes stale by more than 15 every third tile; head 2:
    N(0, 1) scores with one key 300 above the rest (natural units) near the end of each row,
    where the held maximum gives an infinite p."""
    rng = np.random.default_rng(4242)
    B, N, sq, skv, D = 1, 3, 256, 1024, 128
    q = rng.standard_normal((B, N, sq, D)) * 0.05
    k = rng.standard_normal((B, N, skv, D)) * 0.05
    v = rng.standard_normal((B, N, skv, D))
    j = np.arange(skv)
    q[:, :2, :, 0] = 1.0
    k[0, 0, :, 0] = 20 * np.log(2) / 64 * j
    k[0, 1, :, 0] = 6 * np.log(2) / 64 * j
    q[:, 2] = rng.standard_normal((sq, D)) / np.sqrt(D)
    k[:, 2] = rng.standard_normal((skv, D)) / np.sqrt(D)
    q[0, 2, :, 1] = 1.0
    k[0, 2, 900, 1] = 300.0
    q, k, v = (torch.from_numpy(x).to(torch.bfloat16) for x in (q, k, v))
    kw = dict(pre_tokens=1 << 20, next_tokens=1 << 20) if mode == 0 else {}
    o, lse = run(q, k, v, "BNSD", mode, 1.0, gpu_device, **kw)
    ref_o, ref_lse = ref_attention(to64(q), to64(k), to64(v), layout="BNSD", sparse_mode=mode,
                                   scale=1.0, **kw)
    check(o, lse, ref_o, ref_lse, torch.bfloat16, f"row max growth mode {mode}")


def test_softmax_fp16_p_range(gpu_device):
    """fp16 inputs pack P as fp16, whose largest finite value is 65504. Keys 0..63 score 0, so the
    held row maximum after the first tile is 0 (log2 units); key 100 then scores 11.09033203125
    (q = e0 + e1, k = 11.0859375 e0 + 9/2048 e1, scale 1), i.e. p = 2^15.99997 = 65534 against the
    held maximum, and every other key of the second tile scores -50 (p underflows). That lane's
    sum stays below 2^16 with a p that rounds to inf in fp16; the kernel must take the exact update
    for it (its bound is 2^15)."""
    D, sq, skv = 128, 64, 128
    q = np.zeros((1, 1, sq, D))
    k = np.zeros((1, 1, skv, D))
    q[..., 0] = 1.0
    q[..., 1] = 1.0
    k[0, 0, 64:, 0] = -50.0
    k[0, 0, 100, 0] = 11.0859375
    k[0, 0, 100, 1] = 9 / 2048
    v = np.random.default_rng(77).standard_normal((1, 1, skv, D))
    q, k, v = (torch.from_numpy(x).to(torch.float16) for x in (q, k, v))
    kw = dict(pre_tokens=1 << 20, next_tokens=1 << 20)
    o, lse = run(q, k, v, "BNSD", 0, 1.0, gpu_device, **kw)
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    ref_o, ref_lse = ref_attention(to64(q), to64(k), to64(v), layout="BNSD", sparse_mode=0, scale=1.0, **kw)
    check(o, lse, ref_o, ref_lse, torch.float16, "fp16 P range")


# ---------------------------------------------------------------------------------------
# Dense mask (sparseMode=1): the pre-pass tile map and the tile-skipping kernel path
# ---------------------------------------------------------------------------------------

def structured_mask(rng, mb, mh, sq, skv):
    """A uint8 mask (1 = masked) with structure at the kernel's tile scale: 32-row x 64-key
    blocks that are fully masked, fully visible or random; in every other slice the region on
    and below the bottom-right diagonal opened to 90% visible; fully masked rows; and a whole
    256-row q tile with nothing visible. Every tile class and the empty work item occur."""
    m = np.ones((mb, mh, sq, skv), dtype=np.uint8)
    for b in range(mb):
        for h in range(mh):
            for r0 in range(0, sq, 32):
                for c0 in range(0, skv, 64):
                    kind = rng.integers(0, 4)
                    blk = m[b, h, r0:r0 + 32, c0:c0 + 64]
                    if kind == 1:
                        blk[...] = 0
                    elif kind == 2:
                        blk[...] = (rng.random(blk.shape) < 0.5)
            i = np.arange(sq)[:, None]
            j = np.arange(skv)[None, :]
            causal = (j <= i + (skv - sq))
            if (b + h) % 2 == 0:
                m[b, h] &= ~causal.astype(bool) | (rng.random((sq, skv)) < 0.1)
            m[b, h, min(7, sq - 1), :] = 1    # a row that sees nothing
            if sq > 300:
                m[b, h, 256:512, :] = 1       # a q tile with nothing visible
    return m


@pytest.mark.parametrize("bcast", [[0, 0], [1, 0], [0, 1], [1, 1]])
def test_probe_dense_mask_tiles(gpu_device, bcast):
    """Mode-1 tile classes (from the pre-pass the forward runs) against brute force over the
    mask, bit-exact, for aligned (Skv % 16 == 0) and unaligned mask rows."""
    rng = np.random.default_rng(2100 + 2 * bcast[0] + bcast[1])
    B, N = 2, 3
    for sq, skv in [(600, 704), (300, 333), (5, 70)]:
        mb, mh = (1 if bcast[0] else B), (1 if bcast[1] else N)
        mask = structured_mask(rng, mb, mh, sq, skv)
        dims = fb.make_dims(torch.bfloat16, 0, B=B, N=N, Sq=sq, Skv=skv, D=128)
        print(f"[probe-dense] sq={sq} skv={skv} bcast={bcast}", flush=True)
        counts, tiles = fb.fa_mask_probe(dims, "BNSD", 1, device=gpu_device,
                                         atten_mask=torch.from_numpy(mask).to(gpu_device), mask_bcast=bcast)
        torch.cuda.synchronize()
        bm, bn, nq, nk = fb.fa_tile_shape(dims, "BNSD")
        exp = []
        for b in range(B):
            for h in range(N):
                vis = mask[0 if bcast[0] else b, 0 if bcast[1] else h] == 0
                assert counts[b, h].cpu().numpy().tolist() == vis.sum(axis=1).tolist()
                exp += brute_class(vis, bm, bn, nk)
        assert tiles.cpu().numpy().tolist() == exp


@pytest.mark.parametrize("bcast", [[0, 0], [1, 1], [0, 1]])
def test_parity_dense_mask_tiles(gpu_device, bcast):
    """Mode 1 on the MFMA kernel with masks whose tiles are skipped, fully visible or partial,
    empty rows and an empty q tile, against the oracle (bf16 D 128, fp16 D 64; aligned and
    unaligned mask rows; with and without alibi)."""
    rng = np.random.default_rng(2200 + 2 * bcast[0] + bcast[1])
    for dtype, D, layout in [("bf16", 128, "BNSD"), ("f16", 64, "BSND")]:
        for sq, skv in [(600, 704), (300, 333)]:
            B, N = 2, 3
            mb, mh = (1 if bcast[0] else B), (1 if bcast[1] else N)
            mask = structured_mask(rng, mb, mh, sq, skv)
            q, k, v = make_inputs(layout, dtype, B, N, sq, skv, D, seed=2300 + sq)
            for slopes in (None, [0.3, 0.1, 0.02]):
                o, lse = run(q, k, v, layout, 1, 0.1, gpu_device, slopes=slopes, mask=mask, mask_bcast=bcast)
                ref_o, ref_lse = ref_attention(to64(q), to64(k), to64(v), layout=layout, sparse_mode=1, scale=0.1,
                                               atten_mask=mask, alibi_slopes=slopes)
                check(o, lse, ref_o, ref_lse, DT[dtype], f"mode=1 tiles {dtype} {layout} {sq}x{skv} bcast={bcast}")
                zero_rows_ok(o, lse, layout)


def test_dense_mask_equals_causal_mode(gpu_device):
    """"sparseMode介绍": mode 1 fed the boolean mask of mode 3 is mode 3. The MFMA kernel visits
    the same tiles either way, so the results are bitwise equal."""
    for sq, skv in [(700, 700), (333, 600)]:
        q, k, v = make_inputs("BNSD", "bf16", 2, 4, sq, skv, 128, seed=2400 + sq)
        mask = np.triu(np.ones((sq, skv), dtype=np.uint8), 1 + skv - sq)[None, None]
        o1, l1 = run(q, k, v, "BNSD", 1, 0.088, gpu_device, mask=mask, mask_bcast=[1, 1])
        o3, l3 = run(q, k, v, "BNSD", 3, 0.088, gpu_device)
        assert torch.equal(o1, o3) and torch.equal(l1, l3)


@pytest.mark.parametrize("case", ["fixed", "table", "band_empty_items"])
def test_parity_persistent_kernel(gpu_device, monkeypatch, case):
    """The persistent kernel (FA_PERSIST=1: one workgroup per compute unit streaming the K/V
    tiles of several items back to back) against the oracle: fixed-length lists per XCD, the
    varlen / prefix table, items without any visible key (written as empty), several items per
    workgroup (FA_PS_SLOTS=8 forces eight workgroups), alibi, and D 64 / 128."""
    monkeypatch.setenv("FA_PERSIST", "1")
    monkeypatch.setenv("FA_PS_SLOTS", "8")
    if case == "fixed":
        for dtype, D, layout, mode, args in [("bf16", 128, "BNSD", 3, {}), ("f16", 64, "BSND", 4, dict(pre_tokens=70, next_tokens=9)),
                                             ("bf16", 128, "BNSD", 0, dict(pre_tokens=600, next_tokens=-300))]:
            q, k, v = make_inputs(layout, dtype, 2, 4, 700, 650, D, seed=3100 + D)
            for slopes in (None, [0.3, 0.1, 0.02, 0.5]):
                o, lse = run(q, k, v, layout, mode, 0.09, gpu_device, slopes=slopes, **args)
                ref_o, ref_lse = ref_attention(to64(q), to64(k), to64(v), layout=layout, sparse_mode=mode, scale=0.09,
                                               alibi_slopes=slopes, **args)
                check(o, lse, ref_o, ref_lse, DT[dtype], f"persistent {layout} mode={mode} {dtype}")
                zero_rows_ok(o, lse, layout)
    elif case == "table":
        ql, kl = [700, 0, 33, 300, 512, 1], [700, 12, 64, 300, 600, 900]
        q, k, v = make_inputs("TND", "bf16", len(ql), 4, 0, 0, 128, seed=3200, qlens=ql, kvlens=kl)
        cq, ck = synth.cumulative_ends(ql), synth.cumulative_ends(kl)
        o, lse = run(q, k, v, "TND", 3, 0.09, gpu_device, slopes=[0.3, 0.1, 0.02, 0.5], actual_seq_qlen=cq,
                     actual_seq_kvlen=ck)
        ref_o, ref_lse = ref_attention(to64(q), to64(k), to64(v), layout="TND", sparse_mode=3, scale=0.09,
                                       alibi_slopes=[0.3, 0.1, 0.02, 0.5], actual_seq_qlen=cq, actual_seq_kvlen=ck)
        check(o, lse, ref_o, ref_lse, torch.bfloat16, "persistent TND")
        q, k, v = make_inputs("BNSD", "f16", 2, 4, 600, 700, 64, seed=3201)
        o, lse = run(q, k, v, "BNSD", 5, 0.1, gpu_device, prefix=[0, 650])
        ref_o, ref_lse = ref_attention(to64(q), to64(k), to64(v), layout="BNSD", sparse_mode=5, scale=0.1, prefix=[0, 650])
        check(o, lse, ref_o, ref_lse, torch.float16, "persistent prefix")
    else:
        # next = -300: the first q tile of each head sees no key, and whole items are empty.
        q, k, v = make_inputs("BNSD", "bf16", 1, 8, 1100, 1100, 128, seed=3300)
        o, lse = run(q, k, v, "BNSD", 0, 0.09, gpu_device, pre_tokens=2000, next_tokens=-300)
        ref_o, ref_lse = ref_attention(to64(q), to64(k), to64(v), layout="BNSD", sparse_mode=0, scale=0.09,
                                       pre_tokens=2000, next_tokens=-300)
        check(o, lse, ref_o, ref_lse, torch.bfloat16, "persistent empty items")
        zero_rows_ok(o, lse, "BNSD")


@pytest.mark.parametrize("case", ["band", "band_neg", "causal_short", "tnd_band", "band_f16_d64"])
def test_edge_variant_bitwise(gpu_device, monkeypatch, case):
    """The EDGE variant of the ping-pong kernel (a wave that sees nothing of a kv tile skips its
    softmax and hands a zero P^T to its PV product) must give the same bits as the plain kernel:
    such a tile contributes p = 0 and leaves the row's max and sum alone on either path.
    FA_EDGE forces the planner's choice; the plan stats report it."""
    if case == "tnd_band":
        qlens, kvlens = [300, 900, 1200], [300, 1000, 1200]
        q, k, v = make_inputs("TND", "bf16", 3, 4, 0, 0, 128, seed=31, qlens=qlens, kvlens=kvlens)
        kw = dict(layout="TND", mode=0, actual_seq_qlen=synth.cumulative_ends(qlens),
                  actual_seq_kvlen=synth.cumulative_ends(kvlens), pre_tokens=300, next_tokens=0)
    else:
        sq = skv = 1500 if case != "causal_short" else 700
        dt, D = ("f16", 64) if case == "band_f16_d64" else ("bf16", 128)
        q, k, v = make_inputs("BNSD", dt, 2, 4, sq, skv + 37 * (D == 64), D, seed=32)
        kw = {"band": dict(layout="BNSD", mode=4, pre_tokens=300, next_tokens=0),
              "band_neg": dict(layout="BNSD", mode=0, pre_tokens=400, next_tokens=-100),
              "causal_short": dict(layout="BNSD", mode=3),
              "band_f16_d64": dict(layout="BNSD", mode=4, pre_tokens=200, next_tokens=5)}[case]
    layout, mode = kw.pop("layout"), kw.pop("mode")
    outs = []
    for edge in ("0", "1"):
        monkeypatch.setenv("FA_EDGE", edge)
        outs.append(run(q, k, v, layout, mode, 0.088, gpu_device, **kw))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    ref_o, ref_lse = ref_attention(to64(q), to64(k), to64(v), layout=layout, sparse_mode=mode, scale=0.088, **kw)
    check(outs[1][0], outs[1][1], ref_o, ref_lse, q.dtype, f"edge {case}")
