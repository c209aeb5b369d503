"""fa_fwd_noalloc (the workspace in the library's own device array, nothing allocated) against
fa_fwd with a caller-owned workspace, through the C ABI: the same kernels run, so the outputs
must be bitwise equal. Each case makes two calls in a row on the shared array, the second on a
smaller problem, and compares both; the cases cover every use of the workspace (the varlen
and prefix tables, the split-KV decode partials) and a problem that needs none."""

import numpy as np
import pytest
import torch

from masked_attention_forward_amd import binding as fb
from masked_attention_forward_amd import synth

pytestmark = pytest.mark.gpu


def _pair(dev, w, **extra):
    q, k, v = (x.to(dev) for x in w.tensors())
    slopes = torch.tensor(w.slopes(), dtype=torch.float32, device=dev) if w.alibi else None
    kw = dict(layout=w.layout, sparse_mode=w.sparse_mode, pre_tokens=w.pre_tokens, next_tokens=w.next_tokens,
              actual_seq_qlen=w.actual_seq_qlen, actual_seq_kvlen=w.actual_seq_kvlen, prefix=w.prefix,
              alibi_slopes=slopes, scale=w.softmax_scale, **extra)
    print(f"[case] noalloc {w.name} {w.layout} mode={w.sparse_mode} q={tuple(q.shape)} k={tuple(k.shape)}", flush=True)
    out = torch.full_like(q, float("nan"))
    lse = torch.full(fb.lse_shape(q, w.layout), float("nan"), dtype=torch.float32, device=dev)
    fb.fa_fwd_noalloc(q, k, v, out, lse, **kw)
    ref_o, ref_l = fb.flash_attention(q, k, v, **kw)
    return out, lse, ref_o, ref_l


CASES = [
    # (first call, second call on a smaller problem)
    (synth.Workload("varlen", "TND", "bf16", 5, 8, 128, qlens=[700, 0, 33, 300, 512],
                    kvlens=[700, 12, 64, 300, 600], sparse_mode=3, seed=21),
     synth.Workload("varlen_small", "TND", "bf16", 2, 8, 128, qlens=[40, 129], kvlens=[50, 129],
                    sparse_mode=3, seed=22)),
    (synth.Workload("prefix", "BNSD", "f16", 2, 4, 64, 600, 700, sparse_mode=5, prefix=[100, 650],
                    alibi=True, seed=23),
     synth.Workload("prefix_small", "BNSD", "f16", 1, 4, 64, 100, 120, sparse_mode=5, prefix=[7],
                    alibi=True, seed=24)),
    (synth.Workload("decode", "BNSD", "bf16", 3, 8, 128, 1, 20000, sparse_mode=3, seed=25),
     synth.Workload("decode_small", "BNSD", "bf16", 1, 8, 128, 4, 3000, sparse_mode=3, seed=26)),
    (synth.Workload("decode_varlen", "TND", "bf16", 4, 8, 128, qlens=[1, 3, 1, 16],
                    kvlens=[9000, 40, 17000, 5000], sparse_mode=3, seed=27),
     synth.Workload("decode_varlen_small", "TND", "bf16", 2, 8, 128, qlens=[2, 1], kvlens=[2500, 700],
                    sparse_mode=3, seed=28)),
    (synth.Workload("causal", "BSND", "bf16", 2, 4, 128, 500, 500, sparse_mode=3, seed=29),
     synth.Workload("fp32", "BNSD", "f32", 1, 2, 32, 70, 90, sparse_mode=2, seed=30)),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_noalloc_matches_fa_fwd(gpu_device, case):
    for w in CASES[case]:
        out, lse, ref_o, ref_l = _pair(gpu_device, w)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o), w.name
        assert torch.equal(lse, ref_l), w.name
        assert torch.isfinite(out).all(), w.name


def test_noalloc_rejects_oversize(gpu_device):
    """A problem whose workspace exceeds the array is refused with FA_ERR_WORKSPACE and nothing
    is written."""
    n = 600_000   # one-token sequences: a per-batch geometry table of 19 MB
    ql = [1] * n
    dims = fb.make_dims(torch.bfloat16, "TND", B=n, N=1, D=128, T_q=n, T_kv=n)
    need = fb.fa_fwd_workspace_size(dims, "TND", 3, synth.cumulative_ends(ql), synth.cumulative_ends(ql))
    assert need > fb.FA_NOALLOC_SCRATCH_BYTES
    q = torch.zeros(n, 1, 128, dtype=torch.bfloat16, device=gpu_device)
    out = torch.full_like(q, 7.0)
    lse = torch.zeros(1, n, dtype=torch.float32, device=gpu_device)
    with pytest.raises(fb.FaError) as e:
        fb.fa_fwd_noalloc(q, q, q, out, lse, layout="TND", sparse_mode=3, actual_seq_qlen=synth.cumulative_ends(ql),
                          actual_seq_kvlen=synth.cumulative_ends(ql), scale=0.1)
    assert e.value.status == 5
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
