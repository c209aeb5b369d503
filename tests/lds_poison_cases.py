"""Runs a fixed set of forward / backward / decode / paged calls through the library named by
FA_LIBRARY (the normal build or the LDS-poison debug build, see fa_device.h) and prints one
JSON object: per case, a hash of every output's bytes and whether any output holds a NaN.
tests/test_gpu_lds_poison.py runs it once per build and compares the two."""

import hashlib
import json
import os
import sys

import numpy as np
import torch

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
from masked_attention_forward_amd import binding as fb  # noqa: E402
from masked_attention_forward_amd import synth  # noqa: E402

dev = torch.device("cuda:0")
res = {}


def record(name, *ts):
    h = hashlib.sha256()
    nan = False
    for t in ts:
        t = t.detach().contiguous().cpu()
        nan |= bool(torch.isnan(t.float()).any())
        h.update(t.view(torch.uint8).numpy().tobytes() if t.dtype != torch.float32 else t.numpy().tobytes())
    res[name] = {"sha": h.hexdigest()[:20], "nan": nan}


def inputs(layout, dtype, B, N, sq, skv, D, seed, qlens=None, kvlens=None):
    w = synth.Workload("p", layout, dtype, B, N, D, sq, skv, qlens=qlens, kvlens=kvlens, seed=seed)
    return [x.to(dev) for x in w.tensors()]


def fwd(name, q, k, v, layout, mode, **kw):
    print(f"[case] {name}", file=sys.stderr, flush=True)
    o, lse = fb.flash_attention(q, k, v, layout=layout, sparse_mode=mode, scale=0.09, **kw)
    torch.cuda.synchronize()
    record(name, o, lse)
    return o, lse


def fwd_bwd(name, q, k, v, layout, mode, **kw):
    o, lse = fwd(name, q, k, v, layout, mode, **kw)
    do = synth.randn(tuple(q.shape), q.dtype, 123).to(dev)
    dq, dk, dv = fb.flash_attention_backward(q, k, v, o, lse, do, layout=layout, sparse_mode=mode, scale=0.09, **kw)
    torch.cuda.synchronize()
    record(name + "_bwd", dq, dk, dv)


slopes = torch.tensor(synth.alibi_slopes(4), dtype=torch.float32, device=dev)
q, k, v = inputs("BNSD", "bf16", 1, 4, 300, 333, 128, 1)
fwd_bwd("pp_bf16_d128_causal_ragged", q, k, v, "BNSD", 3)
fwd("pp_bf16_d128_band_sqrt_alibi", q, k, v, "BNSD", 4, pre_tokens=100, next_tokens=7, alibi_slopes=slopes,
    alibi_mode="sqrt")
q, k, v = inputs("BSND", "f16", 2, 4, 257, 190, 64, 2)
fwd_bwd("pp_f16_d64_band_negative_next", q, k, v, "BSND", 0, pre_tokens=100, next_tokens=-20)
ql, kl = [0, 70, 129, 1], [5, 70, 300, 64]
q, k, v = inputs("TND", "bf16", len(ql), 4, 0, 0, 128, 3, qlens=ql, kvlens=kl)
fwd_bwd("pp_tnd_empty_sequences", q, k, v, "TND", 3, actual_seq_qlen=synth.cumulative_ends(ql),
        actual_seq_kvlen=synth.cumulative_ends(kl))
q, k, v = inputs("BNSD", "bf16", 2, 4, 200, 330, 128, 4)
rng = np.random.default_rng(5)
m = (rng.random((2, 4, 200, 330)) < 0.7).astype(np.uint8)
m[:, :, 10] = 1          # a fully masked row
m[:, :, :, 64:128] = 1   # a fully masked kv tile
fwd("dense_mask_unbroadcast", q, k, v, "BNSD", 1, atten_mask=torch.from_numpy(m).to(dev), mask_bcast=[0, 0])
fwd("dense_mask_shared", q, k, v, "BNSD", 1, atten_mask=torch.from_numpy(m[:1, :1].copy()).to(dev),
    mask_bcast=[1, 1])
q, k, v = inputs("BNSD", "bf16", 2, 4, 1, 1000, 128, 6)
fwd("decode_one_row", q, k, v, "BNSD", 3)
q, k, v = inputs("BSND", "bf16", 2, 4, 7, 4097, 128, 7)
fwd("decode_spec7_split", q, k, v, "BSND", 3)
# Paged K / V: 64-key pages in reversed order; key rows past the sequence end are NaN in the
# cache and must never reach the output.
q, k, v = inputs("BNSD", "bf16", 1, 4, 200, 300, 128, 8)
bs, npg = 64, 5
bt = torch.tensor([[4, 3, 2, 1, 0]], dtype=torch.int32, device=dev)
caches = []
for x in (k, v):
    c = torch.full((npg, bs, 4, 128), float("nan"), dtype=x.dtype, device=dev)
    seq = x[0].transpose(0, 1)   # [Skv, N, D]
    j = torch.arange(300, device=dev)
    c[bt[0].long()[j // bs], j % bs] = seq
    caches.append(c)
print("[case] paged_nan_tail", file=sys.stderr, flush=True)
o, lse = fb.paged_attention(q, caches[0], caches[1], bt, layout="BNSD", kv_seqlen=300, sparse_mode=3, scale=0.09)
torch.cuda.synchronize()
record("paged_nan_tail", o, lse)
# The four-wave kernel and the persistent kernel on the ragged causal case.
q, k, v = inputs("BNSD", "bf16", 1, 4, 300, 333, 128, 1)
os.environ["FA_KERNEL"] = "mfma32"
fwd("mfma32_causal_ragged", q, k, v, "BNSD", 3)
del os.environ["FA_KERNEL"]
os.environ["FA_PERSIST"], os.environ["FA_PS_SLOTS"] = "1", "2"
fwd("persistent_causal_ragged", q, k, v, "BNSD", 3)
ql, kl = [0, 70, 129, 1], [5, 70, 300, 64]
q, k, v = inputs("TND", "bf16", len(ql), 4, 0, 0, 128, 3, qlens=ql, kvlens=kl)
fwd("persistent_tnd", q, k, v, "TND", 3, actual_seq_qlen=synth.cumulative_ends(ql),
    actual_seq_kvlen=synth.cumulative_ends(kl))
print(json.dumps(res), flush=True)
