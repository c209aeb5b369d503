"""GPU parity at long sequence lengths (sampled rows against the fp64 oracle).

The MFMA kernels address each 64-key tile from a 64-bit base with 32-bit offsets inside the
tile, and the planner splits long kv ranges for decode; these cases reach far past the benchmark
sizes: a 32768 x 32768 BSND prefill (row stride N * D, 256 q tiles of 128 kv tiles each), a
one-row decode over 2^20 keys (many splits and a merge), and a varlen batch mixing a 500000-key
sequence with short ones.
"""

import numpy as np
import pytest
import torch

import oracle
from masked_attention_forward_amd import synth

from test_gpu_parity import check, make_inputs, run

pytestmark = pytest.mark.gpu


def _sampled(q, k, v, layout, mode, scale, rows, got_o, got_l, dtype, what, **kw):
    qn, kn, vn = (x.float().numpy() for x in (q, k, v))
    ref_o, ref_l = oracle.attention_rows(qn, kn, vn, rows, layout=layout, sparse_mode=mode, scale=scale, **kw)
    check(torch.from_numpy(got_o), torch.from_numpy(got_l), ref_o, ref_l, dtype, what)


def test_long_prefill_bsnd(gpu_device):
    """rightDownCausal and a right-down band, BSND bf16, Sq = Skv = 32768, N = 4."""
    B, N, S, D = 1, 4, 32768, 128
    q, k, v = make_inputs("BSND", "bf16", B, N, S, S, D, seed=901)
    rng = np.random.default_rng(5)
    idx = sorted({0, 1, 255, 256, 4095, S - 1} | set(int(x) for x in rng.integers(0, S, 10)))
    for mode, kw in [(3, {}), (4, dict(pre_tokens=3000, next_tokens=0))]:
        o, lse = run(q, k, v, "BSND", mode, 0.0884, gpu_device, **kw)
        assert torch.isfinite(o).all()
        rows = [(0, h, i) for h in (0, N - 1) for i in idx]
        got_o = np.array([o[0, i, h].double().numpy() for _, h, i in rows])
        got_l = np.array([float(lse[0, h, i]) for _, h, i in rows])
        _sampled(q, k, v, "BSND", mode, 0.0884, rows, got_o, got_l, torch.bfloat16, f"BSND 32768 mode {mode}", **kw)


def test_long_decode_one_million_keys(gpu_device):
    """One query row over 2^20 keys per head (BNSD bf16, two heads)."""
    B, N, Skv, D = 1, 2, 1 << 20, 128
    q, k, v = make_inputs("BNSD", "bf16", B, N, 1, Skv, D, seed=902)
    o, lse = run(q, k, v, "BNSD", 3, 0.0884, gpu_device)
    rows = [(0, h, 0) for h in range(N)]
    got_o = np.array([o[0, h, 0].double().numpy() for h in range(N)])
    got_l = np.array([float(lse[0, h, 0]) for h in range(N)])
    _sampled(q, k, v, "BNSD", 3, 0.0884, rows, got_o, got_l, torch.bfloat16, "decode 2^20 keys")


def test_long_varlen_tnd(gpu_device):
    """TND bf16 with one 500000-key sequence among short ones (more than 16 rows: prefill kernel)."""
    ql = [1, 20000, 3, 64]
    kl = [500000, 20000, 70000, 64]
    N, D = 2, 128
    q, k, v = make_inputs("TND", "bf16", len(ql), N, 0, 0, D, seed=903, qlens=ql, kvlens=kl)
    cq, ck = synth.cumulative_ends(ql), synth.cumulative_ends(kl)
    kw = dict(actual_seq_qlen=cq, actual_seq_kvlen=ck)
    o, lse = run(q, k, v, "TND", 3, 0.0884, gpu_device, **kw)
    rng = np.random.default_rng(6)
    rows = [(0, 0, 0), (0, 1, 0), (2, 0, 2), (3, 1, 63)]
    rows += [(1, int(rng.integers(0, N)), int(i)) for i in [0, 19999] + list(rng.integers(0, 20000, 6))]
    starts = [0] + cq[:-1]
    got_o = np.array([o[starts[b] + i, h].double().numpy() for b, h, i in rows])
    got_l = np.array([float(lse[h, starts[b] + i]) for b, h, i in rows])
    _sampled(q, k, v, "TND", 3, 0.0884, rows, got_o, got_l, torch.bfloat16, "TND long", **kw)
