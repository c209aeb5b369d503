"""GPU parity of the paged forward (fa_fwd_paged, through the C ABI): K and V read from
"Norm" / "NHSD" caches ("aclnnScatterPaKvCache", scenarios two and seven) through a block
table, against the fp64 oracle on the dense K / V.

Every case builds its caches from seeded dense K / V with plain indexing, checks that the
oracle's block-table read-back (kv_cache.gather_paged, pinned in the oracle tests) returns
exactly those K / V, and compares the library with the oracle at the forward pass's
tolerances. When the paged call and fa_fwd on the dense K / V run the same kernel, their
outputs must also agree bit for bit (only addresses differ).
"""

import math

import numpy as np
import pytest
import torch

import oracle
from masked_attention_forward_amd import binding as fb
from masked_attention_forward_amd import synth
from oracle import kv_cache

from test_gpu_parity import DT, check, make_inputs, to64, zero_rows_ok

pytestmark = pytest.mark.gpu


def bits(t):
    return t.contiguous().view({2: torch.int16, 4: torch.int32}[t.element_size()]).cpu().numpy()


def seqs_of(x, layout, ends=None):
    """Per-sequence [L, N, D] views of a K or V tensor in `layout`."""
    if layout == "BNSD":
        return [x[b].transpose(0, 1) for b in range(x.shape[0])]
    if layout == "BSND":
        return [x[b] for b in range(x.shape[0])]
    starts = [0] + list(ends[:-1])
    return [x[s:e] for s, e in zip(starts, ends)]


def make_table(lens, nb, bs, rng, pad=2):
    """Block table [B, max_pages + pad]: distinct random pages for every sequence; entries past
    a sequence's last page hold ids that are never read (large, outside the cache)."""
    need = [-(-L // bs) for L in lens]
    assert sum(need) <= nb
    perm = rng.permutation(nb)
    width = max(need + [0]) + pad
    bt = rng.integers(nb, 1 << 30, size=(len(lens), width)).astype(np.int32)
    p = 0
    for b, n in enumerate(need):
        bt[b, :n] = perm[p:p + n]
        p += n
    return bt


def fill_cache(seqs, bt, nb, bs, layout, dtype, device, seed):
    """A cache whose unused slots hold random values, with sequence b's key j at page
    bt[b, j // bs], offset j % bs."""
    N, D = seqs[0].shape[1], seqs[0].shape[2]
    gen = torch.Generator().manual_seed(seed)
    shape = (nb, bs, N, D) if layout == "Norm" else (nb, N, bs, D)
    cache = (3 * torch.randn(*shape, generator=gen)).to(dtype).to(device)
    view = cache if layout == "Norm" else cache.permute(0, 2, 1, 3)   # [nb, bs, N, D]
    for b, s in enumerate(seqs):
        L = s.shape[0]
        if L == 0:
            continue
        j = torch.arange(L)
        pages = torch.from_numpy(bt[b].astype(np.int64))[j // bs]
        view[pages.to(device), (j % bs).to(device)] = s.to(device=device, dtype=dtype)
    return cache


def check_readback(cache, bt, seqs, layout):
    """The oracle's block-table read of the cache gives back the dense sequences exactly."""
    c = bits(cache)
    for b, s in enumerate(seqs):
        got = kv_cache.gather_paged(c, bt[b], s.shape[0], layout)
        assert np.array_equal(got, bits(s)), f"read-back of sequence {b}"


def pp_kernel(dtype, D, mode, bs, max_len):
    """Whether fa_fwd (dense) and fa_fwd_paged pick the ping-pong kernel (paged: pages of a
    power of two >= 64 keys, at most 2048 of them per sequence, no explicit mask)."""
    dense = DT[dtype] in (torch.float16, torch.bfloat16) and D in (64, 128)
    paged = dense and mode != 1 and bs >= 64 and bs & (bs - 1) == 0 and -(-max_len // bs) <= 2048
    return dense, paged


def run_case(dev, layout, dtype, D, mode, bs, cache_layout, *, B=2, N=3, sq=300, skv=333, qlens=None, kvlens=None,
             slopes=None, alibi_mode="right", mask=None, mask_bcast=None, seed=0, bad_page=None, readback=True,
             **args):
    if layout == "TND":
        B = len(qlens)
    q, k, v = make_inputs(layout, dtype, B, N, sq, skv, D, seed=seed, qlens=qlens, kvlens=kvlens)
    ends = kw_q = kw_kv = None
    if layout == "TND":
        kw_q, kw_kv = synth.cumulative_ends(qlens), synth.cumulative_ends(kvlens)
        ends = kw_kv
    ks, vs = seqs_of(k, layout, ends), seqs_of(v, layout, ends)
    lens = [s.shape[0] for s in ks]
    rng = np.random.default_rng(seed + 1)
    nb = sum(-(-L // bs) for L in lens) + 5
    bt = make_table(lens, nb, bs, rng)
    kc = fill_cache(ks, bt, nb, bs, cache_layout, DT[dtype], dev, seed + 2)
    vc = fill_cache(vs, bt, nb, bs, cache_layout, DT[dtype], dev, seed + 3)
    if readback:
        check_readback(kc, bt, ks, cache_layout)
        check_readback(vc, bt, vs, cache_layout)
    k_ref, v_ref = k, v
    if bad_page is not None:
        # page id outside the cache: its keys read as zeros
        b, idx = bad_page
        bt[b, idx] = -1 if idx % 2 == 0 else nb + 3
        k_ref, v_ref = k.clone(), v.clone()
        for t in (k_ref, v_ref):
            for s_ in seqs_of(t, layout, ends)[b:b + 1]:
                s_[idx * bs:(idx + 1) * bs] = 0
    sl = torch.tensor(slopes, dtype=torch.float32, device=dev) if slopes is not None else None
    md = torch.from_numpy(np.ascontiguousarray(mask)).to(dev) if mask is not None else None
    kw = dict(args)
    if layout == "TND":
        kw.update(actual_seq_qlen=kw_q, actual_seq_kvlen=kw_kv)
    print(f"[case] paged {layout} {cache_layout} {dtype} D={D} bs={bs} mode={mode} q={tuple(q.shape)} "
          f"lens={lens if len(lens) < 10 else len(lens)} alibi={alibi_mode if slopes else None} bad={bad_page} "
          f"{ {a: c for a, c in args.items()} }", flush=True)
    qd = q.to(dev)
    o, lse = fb.paged_attention(qd, kc, vc, torch.from_numpy(bt).to(dev), layout=layout, cache_layout=cache_layout,
                                kv_seqlen=skv if layout != "TND" else 0, sparse_mode=mode,
                                scale=1.0 / math.sqrt(D), alibi_slopes=sl, alibi_mode=alibi_mode, atten_mask=md,
                                mask_bcast=mask_bcast, **kw)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    ref_o, ref_lse = oracle.attention(to64(q), to64(k_ref), to64(v_ref), layout=layout, sparse_mode=mode,
                                      scale=1.0 / math.sqrt(D), alibi_slopes=slopes, alibi_mode=alibi_mode,
                                      atten_mask=mask, **kw)
    what = f"paged {layout}/{cache_layout} {dtype} D={D} bs={bs} mode={mode} {args}"
    check(o, lse, ref_o, ref_lse, DT[dtype], what)
    zero_rows_ok(o, lse, layout)
    dense_pp, paged_pp = pp_kernel(dtype, D, mode, bs, max(lens))
    if dense_pp == paged_pp and bad_page is None:
        o2, lse2 = fb.flash_attention(qd, k.to(dev), v.to(dev), layout=layout, sparse_mode=mode,
                                      scale=1.0 / math.sqrt(D), alibi_slopes=sl, alibi_mode=alibi_mode,
                                      atten_mask=md, mask_bcast=mask_bcast, **kw)
        torch.cuda.synchronize()
        assert torch.equal(o2.cpu(), o) and torch.equal(lse2.cpu(), lse), f"{what}: differs from fa_fwd"
    return o, lse


# (dtype, D, page size): the first three run the ping-pong kernel, the rest the generic one
PAGE_VARIANTS = [("bf16", 128, 64), ("bf16", 128, 128), ("f16", 64, 256), ("bf16", 128, 16), ("f32", 32, 16),
                 ("f16", 64, 48)]
MODES = [(0, dict(pre_tokens=40, next_tokens=25)), (3, {}), (4, dict(pre_tokens=60, next_tokens=7)),
         (5, dict(prefix=[250, 10]))]


@pytest.mark.parametrize("cache_layout", ["Norm", "NHSD"])
@pytest.mark.parametrize("variant", range(len(PAGE_VARIANTS)))
def test_paged_parity_bnsd_bsnd(gpu_device, cache_layout, variant):
    dtype, D, bs = PAGE_VARIANTS[variant]
    for mi, (mode, args) in enumerate(MODES):
        layout = "BNSD" if mi % 2 == 0 else "BSND"
        slopes = synth.alibi_slopes(3) if mi == 1 else None
        run_case(gpu_device, layout, dtype, D, mode, bs, cache_layout, slopes=slopes,
                 seed=100 * variant + 10 * mi, **args)


@pytest.mark.parametrize("cache_layout", ["Norm", "NHSD"])
@pytest.mark.parametrize("mode", [3, 5, 7, 8])
def test_paged_parity_tnd(gpu_device, cache_layout, mode):
    """Varlen TND with empty sequences, single-key sequences and lengths off the page grid."""
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
    for dtype, D, bs in [("bf16", 128, 64), ("f16", 64, 128), ("f32", 32, 16)]:
        run_case(gpu_device, "TND", dtype, D, mode, bs, cache_layout, N=4, qlens=ql, kvlens=kl, slopes=slopes,
                 seed=500 + mode + D, **kw)


@pytest.mark.parametrize("alibi_mode", ["sqrt", "left"])
def test_paged_alibi_variants(gpu_device, alibi_mode):
    for dtype, D, bs in [("bf16", 128, 128), ("f32", 32, 16)]:
        run_case(gpu_device, "BNSD", dtype, D, 4, bs, "Norm", slopes=[0.6, 0.25, 0.05], alibi_mode=alibi_mode,
                 seed=900 + D, pre_tokens=60, next_tokens=7)


def test_paged_dense_mask(gpu_device):
    """An explicit mask (sparse mode 1) with paged K / V: the generic kernel."""
    rng = np.random.default_rng(61)
    mask = (rng.random((1, 3, 150, 170)) < 0.7).astype(np.uint8)
    mask[..., 5, :] = 1
    for dtype, D, bs in [("bf16", 128, 64), ("f32", 32, 16)]:
        run_case(gpu_device, "BNSD", dtype, D, 1, bs, "NHSD", sq=150, skv=170, mask=mask, mask_bcast=[1, 0],
                 seed=61 + D)


@pytest.mark.parametrize("bs", [64, 16])
def test_paged_invalid_page_reads_zeros(gpu_device, bs):
    """A page id outside [0, num_blocks) is never dereferenced: its keys read as zeros."""
    run_case(gpu_device, "BNSD", "bf16", 128, 3, bs, "Norm", seed=77, bad_page=(1, 2))
    run_case(gpu_device, "BNSD", "bf16", 128, 3, bs, "NHSD", seed=78, bad_page=(0, 3))


def test_paged_long_sequence_many_pages(gpu_device):
    """2048 pages of 64 keys in one sequence (the largest page table the ping-pong kernel
    stages), and one past it (generic kernel)."""
    for skv in (2048 * 64, 2048 * 64 + 1):
        run_case(gpu_device, "BNSD", "bf16", 128, 3, 64, "Norm", B=1, N=1, sq=300, skv=skv, seed=88,
                 readback=False)


def test_scatter_then_paged_matches_dense(gpu_device):
    """The serving flow: fa_scatter_kv_cache writes each token's K / V at its slot
    (page * block_size + offset, pages from the block table), then fa_fwd_paged reads them
    back; bitwise equal to fa_fwd on the dense K / V."""
    B, N, S, D, bs = 3, 8, 1000, 128, 128
    q, k, v = make_inputs("BSND", "bf16", B, N, S, S, D, seed=1234)
    rng = np.random.default_rng(1234)
    nb = B * (-(-S // bs)) + 7
    bt = make_table([S] * B, nb, bs, rng)
    j = np.arange(S)
    slots = np.concatenate([bt[b, j // bs].astype(np.int64) * bs + j % bs for b in range(B)])
    dev = gpu_device
    for cache_layout in ("Norm", "NHSD"):
        shape = (nb, bs, N, D) if cache_layout == "Norm" else (nb, N, bs, D)
        kc = torch.zeros(shape, dtype=torch.bfloat16, device=dev)
        vc = torch.zeros(shape, dtype=torch.bfloat16, device=dev)
        fb.fa_scatter_kv_cache(k.reshape(B * S, N, D).to(dev), kc, torch.from_numpy(slots).to(dev),
                               v.reshape(B * S, N, D).to(dev), vc, layout=cache_layout)
        o, lse = fb.paged_attention(q.to(dev), kc, vc, torch.from_numpy(bt).to(dev), layout="BSND",
                                    cache_layout=cache_layout, kv_seqlen=S, sparse_mode=3, scale=0.0884)
        o2, lse2 = fb.flash_attention(q.to(dev), k.to(dev), v.to(dev), layout="BSND", sparse_mode=3, scale=0.0884)
        torch.cuda.synchronize()
        assert torch.equal(o, o2) and torch.equal(lse, lse2), cache_layout


@pytest.mark.parametrize("cache_layout", ["Norm", "NHSD"])
def test_paged_full_size_matches_dense(gpu_device, cache_layout):
    """The rightDownCausal 2 x 32 x 8192 x 128 bf16 workload from 128-key pages: bitwise equal
    to fa_fwd on the dense K / V, whose sampled rows the oracle checks in the parity tests."""
    w = synth.workloads()["causal_8192"]
    q, k, v = w.tensors()
    dev = gpu_device
    print(f"[case] paged full size {cache_layout} {w.layout} {tuple(q.shape)}", flush=True)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    bs = 128
    rng = np.random.default_rng(8192)
    nb = w.B * w.Skv // bs + 3
    bt = make_table([w.Skv] * w.B, nb, bs, rng)
    kc = fill_cache(seqs_of(kd, w.layout), bt, nb, bs, cache_layout, torch.bfloat16, dev, 1)
    vc = fill_cache(seqs_of(vd, w.layout), bt, nb, bs, cache_layout, torch.bfloat16, dev, 2)
    o, lse = fb.paged_attention(qd, kc, vc, torch.from_numpy(bt).to(dev), layout=w.layout,
                                cache_layout=cache_layout, kv_seqlen=w.Skv, sparse_mode=w.sparse_mode,
                                scale=w.softmax_scale)
    o2, lse2 = fb.flash_attention(qd, kd, vd, layout=w.layout, sparse_mode=w.sparse_mode, scale=w.softmax_scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


@pytest.mark.parametrize("case", ["band", "causal_short"])
def test_paged_edge_variant_bitwise(gpu_device, monkeypatch, case):
    """The paged ping-pong kernel's EDGE variant (a wave that sees nothing of a kv tile skips its
    softmax) gives the same bits as the plain paged kernel and as the dense forward on the same
    K / V, read from 128-key pages in a random order. FA_EDGE forces the planner's choice."""
    B, N, S, D, bs = 2, 4, 1500 if case == "band" else 700, 128, 128
    q, k, v = make_inputs("BSND", "bf16", B, N, S, S, D, seed=4321)
    rng = np.random.default_rng(4321)
    nb = B * (-(-S // bs)) + 5
    bt = make_table([S] * B, nb, bs, rng)
    dev = gpu_device
    kc = fill_cache(seqs_of(k, "BSND"), bt, nb, bs, "Norm", torch.bfloat16, dev, seed=1)
    vc = fill_cache(seqs_of(v, "BSND"), bt, nb, bs, "Norm", torch.bfloat16, dev, seed=2)
    kw = dict(sparse_mode=4, pre_tokens=300, next_tokens=0) if case == "band" else dict(sparse_mode=3)
    print(f"[case] paged edge {case} S={S}", flush=True)
    outs = []
    for edge in ("0", "1"):
        monkeypatch.setenv("FA_EDGE", edge)
        outs.append(fb.paged_attention(q.to(dev), kc, vc, torch.from_numpy(bt).to(dev), layout="BSND",
                                       cache_layout="Norm", kv_seqlen=S, scale=0.0884, **kw))
    dense = fb.flash_attention(q.to(dev), k.to(dev), v.to(dev), layout="BSND", scale=0.0884, **kw)
    torch.cuda.synchronize()
    for o, lse in outs[1:] + [dense]:
        assert torch.equal(outs[0][0], o) and torch.equal(outs[0][1], lse)
