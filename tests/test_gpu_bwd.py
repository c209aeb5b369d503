"""GPU parity of the backward pass (fa_bwd, through the C ABI) against the fp64 oracle
(oracle.backward, pinned against float64 autograd and finite differences).

Each case runs fa_fwd for out and softmax_lse, then fa_bwd with a seeded dO, and compares
dQ, dK and dV element by element with the oracle's gradients of the same inputs.

Tolerances. With fp32 inputs nothing is rounded below fp32: |d| <= 1e-4 * max(1, max|ref|)
per tensor (fp32 sums of up to a few thousand terms). With fp16 / bf16 inputs P and dS are
rounded to the input type before the products that consume them (relative 2^-9 for bf16),
the forward's O that Delta is computed from is rounded, and the gradients are rounded on
output: |d| <= 2e-2 * max|ref| + 2e-2 * |ref| per tensor, with the mean error also below
2e-3 * max|ref|.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from masked_attention_forward_amd import binding as fb
from masked_attention_forward_amd import synth

from test_gpu_parity import DT, make_inputs, to64

pytestmark = pytest.mark.gpu


def check_grad(got, ref, dtype, what):
    got = to64(got)
    assert got.shape == ref.shape, what
    if ref.size == 0:
        return
    assert np.isfinite(got).all(), f"{what}: non-finite gradient"
    scale = max(1.0, float(np.abs(ref).max(initial=0.0)))
    err = np.abs(got - ref)
    if dtype == torch.float32:
        assert err.max(initial=0.0) <= 1e-4 * scale, f"{what}: max |d| {err.max()} (scale {scale})"
        return
    bound = 2e-2 * scale + 2e-2 * np.abs(ref)
    bad = err > bound
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} out of tolerance, max |d| {err.max()} (scale {scale})"
    assert err.mean() <= 2e-3 * scale, f"{what}: mean |d| {err.mean()} (scale {scale})"
    print(f"[err] {what}: max {err.max() / scale:.2e}, mean {err.mean() / scale:.2e} of scale {scale:.3g}")


def bwd_case(dev, layout, dtype, D, mode, sq, skv, *, B=2, N=3, qlens=None, kvlens=None, slopes=None,
             alibi_mode="right", mask=None, mask_bcast=None, seed=0, misalign_out=False, **kw):
    if layout == "TND":
        B = len(qlens)
        kw.update(actual_seq_qlen=synth.cumulative_ends(qlens), actual_seq_kvlen=synth.cumulative_ends(kvlens))
    q, k, v = make_inputs(layout, dtype, B, N, sq, skv, D, seed=seed, qlens=qlens, kvlens=kvlens)
    do = synth.randn(tuple(q.shape), DT[dtype], seed + 77)
    scale = 1.0 / math.sqrt(D)
    sl = torch.tensor(slopes, dtype=torch.float32, device=dev) if slopes is not None else None
    md = torch.from_numpy(np.ascontiguousarray(mask)).to(dev) if mask is not None else None
    print(f"[case] bwd {layout} {dtype} D={D} mode={mode} q={tuple(q.shape)} k={tuple(k.shape)} "
          f"alibi={alibi_mode if slopes else None} {kw if len(str(kw)) < 200 else ''}", flush=True)
    qd, kd, vd, dod = (x.to(dev) for x in (q, k, v, do))
    out, lse = fb.flash_attention(qd, kd, vd, layout=layout, sparse_mode=mode, scale=scale, alibi_slopes=sl,
                                  alibi_mode=alibi_mode, atten_mask=md, mask_bcast=mask_bcast, **kw)
    if misalign_out:
        # The same O, one element past a 16-byte boundary.
        buf = torch.empty(out.numel() + 1, dtype=out.dtype, device=dev)
        moved = buf[1:].view(out.shape)
        moved.copy_(out)
        out = moved
        assert out.data_ptr() % 16 != 0
    dq, dk, dv = fb.flash_attention_backward(qd, kd, vd, out, lse, dod, layout=layout, sparse_mode=mode, scale=scale,
                                             alibi_slopes=sl, alibi_mode=alibi_mode, atten_mask=md,
                                             mask_bcast=mask_bcast, **kw)
    torch.cuda.synchronize()
    ref = oracle.attention_backward(to64(q), to64(k), to64(v), to64(do), layout=layout, sparse_mode=mode,
                                    scale=scale, alibi_slopes=slopes, alibi_mode=alibi_mode, atten_mask=mask, **kw)
    what = f"{layout} {dtype} D={D} mode={mode}"
    for name, got, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        check_grad(got.cpu(), r, DT[dtype], f"{what} {name}")
    return dq, dk, dv


VARIANTS = [("bf16", 128, "BNSD"), ("f16", 64, "BSND"), ("f32", 32, "BNSD"), ("bf16", 40, "BSND")]
MODES = [(0, dict(pre_tokens=100, next_tokens=20)), (0, dict(pre_tokens=400, next_tokens=-30)), (2, {}), (3, {}),
         (4, dict(pre_tokens=90, next_tokens=5)), (5, dict(prefix=[150, 3]))]


@pytest.mark.parametrize("variant", range(len(VARIANTS)))
@pytest.mark.parametrize("mode_i", range(len(MODES)))
def test_bwd_parity(gpu_device, variant, mode_i):
    """MFMA kernels (bf16 D 128, fp16 D 64) and generic ones (fp32, D 40), ragged tiles with
    Sq and Skv on both sides of each other."""
    dtype, D, layout = VARIANTS[variant]
    mode, args = MODES[mode_i]
    for sq, skv in [(300, 333), (130, 200), (200, 77)]:
        if mode == 0 and args.get("next_tokens", 0) < 0 and -args["next_tokens"] >= skv:
            continue
        bwd_case(gpu_device, layout, dtype, D, mode, sq, skv, seed=10 * variant + mode_i + sq, **args)


@pytest.mark.parametrize("alibi_mode", ["right", "sqrt", "left"])
def test_bwd_alibi(gpu_device, alibi_mode):
    for dtype, D, layout in [("bf16", 128, "BNSD"), ("f16", 64, "BSND"), ("f32", 32, "BNSD")]:
        for mode, args in [(3, {}), (4, dict(pre_tokens=60, next_tokens=7)), (5, dict(prefix=[200, 10]))]:
            bwd_case(gpu_device, layout, dtype, D, mode, 260, 300, slopes=[0.6, 0.25, 0.05], alibi_mode=alibi_mode,
                     seed=900 + D + mode, **args)


def test_bwd_delta_paths(gpu_device):
    """Delta = rowsum(dO * O) has a 16-byte vector kernel for fp16 / bf16 and a scalar one for the
    rest. Two-byte cases that take the scalar kernel: D not a multiple of 8 (bf16 D 36), and an O
    whose base is not 16-byte aligned (bf16 D 128, fp16 D 64)."""
    bwd_case(gpu_device, "BNSD", "bf16", 36, 3, 130, 150, seed=81)
    bwd_case(gpu_device, "BNSD", "bf16", 128, 3, 130, 150, seed=82, misalign_out=True)
    bwd_case(gpu_device, "BSND", "f16", 64, 4, 200, 180, seed=83, misalign_out=True, pre_tokens=50, next_tokens=10)


def test_bwd_dense_mask(gpu_device):
    rng = np.random.default_rng(71)
    for dtype, D, layout in [("bf16", 128, "BNSD"), ("f32", 32, "BSND")]:
        mask = (rng.random((1, 3, 150, 170)) < 0.6).astype(np.uint8)
        mask[..., 5, :] = 1   # a row that sees nothing
        bwd_case(gpu_device, layout, dtype, D, 1, 150, 170, mask=mask, mask_bcast=[1, 0], seed=71)


@pytest.mark.parametrize("mode", [3, 5, 7, 8])
def test_bwd_tnd(gpu_device, mode):
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
        kw = dict(prefix=[0, 3, 9, 200, 64, 400])
    slopes = synth.alibi_slopes(4) if mode in (3, 5) else None
    for dtype, D in [("bf16", 128), ("f16", 64), ("f32", 32)]:
        bwd_case(gpu_device, "TND", dtype, D, mode, 0, 0, N=4, qlens=ql, kvlens=kl, slopes=slopes, seed=500 + mode,
                 **kw)


def test_bwd_empty_and_degenerate(gpu_device):
    """No query rows (dK = dV = 0), no keys (dQ = 0), a single key, a single row."""
    for sq, skv in [(0, 50), (40, 0), (7, 1), (1, 90)]:
        for dtype, D in [("bf16", 128), ("f32", 32)]:
            bwd_case(gpu_device, "BNSD", dtype, D, 2 if skv == 1 else 3, sq, skv, seed=40 + sq + skv)


def test_bwd_deterministic(gpu_device):
    q, k, v = make_inputs("BNSD", "bf16", 2, 4, 500, 500, 128, seed=3)
    do = synth.randn(tuple(q.shape), torch.bfloat16, 5)
    qd, kd, vd, dod = (x.to(gpu_device) for x in (q, k, v, do))
    out, lse = fb.flash_attention(qd, kd, vd, sparse_mode=3, scale=0.088)
    g1 = fb.flash_attention_backward(qd, kd, vd, out, lse, dod, sparse_mode=3, scale=0.088)
    g2 = fb.flash_attention_backward(qd, kd, vd, out, lse, dod, sparse_mode=3, scale=0.088)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_bwd_full_size_heads(gpu_device):
    """The rightDownCausal 2 x 32 x 8192 x 128 bf16 workload: two whole (batch, head) slices of
    the full-size launch against the oracle."""
    w = synth.workloads()["causal_8192"]
    q, k, v = w.tensors()
    do = synth.randn(tuple(q.shape), torch.bfloat16, 8080)
    qd, kd, vd, dod = (x.to(gpu_device) for x in (q, k, v, do))
    out, lse = fb.flash_attention(qd, kd, vd, sparse_mode=3, scale=w.softmax_scale)
    dq, dk, dv = fb.flash_attention_backward(qd, kd, vd, out, lse, dod, sparse_mode=3, scale=w.softmax_scale)
    torch.cuda.synchronize()
    for b, h in [(0, 0), (1, 31)]:
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref = oracle.attention_backward(to64(q[sl]), to64(k[sl]), to64(v[sl]), to64(do[sl]), layout="BNSD",
                                        sparse_mode=3, scale=w.softmax_scale)
        for name, got, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
            check_grad(got[sl].cpu(), r, torch.bfloat16, f"causal_8192 b={b} h={h} {name}")


def test_bwd_delta_values(gpu_device):
    """Delta = rowsum(dO * O), read back from a caller-owned workspace and compared with an fp64
    sum of the same two rounded tensors, for the 16-byte vector kernel (BNSD, BSND, TND) and the
    scalar one (D not a multiple of 8; an O that is not 16-byte aligned). Delta lives where the
    library puts it: laid out like softmax_lse, at offset 0, or after the per-batch geometry
    table (B entries of 32 bytes, rounded up to 256) in TND and prefix modes.

    Bound: the products of two 16-bit floats are exact in fp32; a sum of D of them in fp32 is
    within D 2^-24 of the sum of their magnitudes, so |d| <= 2^-17 sum|dO O| with D <= 128."""
    cases = [("BNSD", "bf16", 128, False), ("BSND", "f16", 64, False), ("TND", "bf16", 128, False),
             ("BNSD", "bf16", 36, False), ("BNSD", "bf16", 128, True)]
    for layout, dtype, D, misalign in cases:
        qlens = kvlens = None
        kw = {}
        B, N, sq, skv = 2, 3, 150, 170
        if layout == "TND":
            qlens, kvlens = [100, 0, 37], [120, 9, 37]
            B = len(qlens)
            kw = dict(actual_seq_qlen=synth.cumulative_ends(qlens), actual_seq_kvlen=synth.cumulative_ends(kvlens))
        q, k, v = make_inputs(layout, dtype, B, N, sq, skv, D, seed=600 + D, qlens=qlens, kvlens=kvlens)
        do = synth.randn(tuple(q.shape), DT[dtype], 601 + D)
        qd, kd, vd, dod = (x.to(gpu_device) for x in (q, k, v, do))
        print(f"[case] delta {layout} {dtype} D={D} misaligned O={misalign}", flush=True)
        out, lse = fb.flash_attention(qd, kd, vd, layout=layout, sparse_mode=3, scale=0.1, **kw)
        if misalign:
            buf = torch.empty(out.numel() + 1, dtype=out.dtype, device=gpu_device)
            moved = buf[1:].view(out.shape)
            moved.copy_(out)
            out = moved
            assert out.data_ptr() % 16 != 0
        dims = fb.dims_of(qd, kd, layout, kw.get("actual_seq_qlen"))
        ws_bytes = fb.fa_bwd_workspace_size(dims, layout, 3, kw.get("actual_seq_qlen"), kw.get("actual_seq_kvlen"))
        ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=gpu_device)
        dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
        fb.fa_bwd(qd, kd, vd, out, lse, dod, dq, dk, dv, layout=layout, sparse_mode=3, scale=0.1, workspace=ws, **kw)
        torch.cuda.synchronize()
        off = ((B * 32 + 255) // 256) * 256 if layout == "TND" else 0
        n = lse.numel()
        delta = ws[off:off + 4 * n].cpu().view(torch.float32).reshape(lse.shape).double().numpy()
        prod = to64(dod) * to64(out)
        ref, mag = prod.sum(-1), np.abs(prod).sum(-1)
        if layout == "BSND":
            ref, mag = ref.transpose(0, 2, 1), mag.transpose(0, 2, 1)
        if layout == "TND":
            ref, mag = ref.T, mag.T
        err = np.abs(delta - ref)
        assert (err <= 2.0 ** -17 * mag + 1e-30).all(), f"{layout} {dtype} D={D}: max |d| {err.max()}"
