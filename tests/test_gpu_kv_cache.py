"""GPU parity of the paged KV cache scatter (libfa.so, through its C ABI) against the oracle:
bit-exact, since it is pure data movement ("aclnnScatterPaKvCache", scenarios two, six and
seven)."""

import numpy as np
import pytest
import torch

from masked_attention_forward_amd import binding as fb
from oracle import kv_cache

pytestmark = pytest.mark.gpu


def bits(t):
    """Raw element bits as a numpy integer array (the scatter moves bytes, not values)."""
    return t.view({1: torch.int8, 2: torch.int16, 4: torch.int32}[t.element_size()]).numpy()


def _case(gpu_device, layout, dtype, T, N, dk, dv, nb, bs, slot_dtype, seed, with_value=True, bad_slots=0):
    rng = np.random.default_rng(seed)
    gen = torch.Generator().manual_seed(seed)

    def rnd(*shape):
        if dtype in (torch.int8, torch.int32):
            return torch.randint(-100, 100, shape, generator=gen, dtype=dtype)
        return torch.randn(*shape, generator=gen).to(dtype)

    slots = rng.permutation(nb * bs)[:T].astype(np.int64)
    if bad_slots:
        slots[:bad_slots] = rng.choice([-1, nb * bs, nb * bs + 7], bad_slots)
    key, val = rnd(T, N, dk), rnd(T, N, dv)
    kshape = (nb, bs, N, dk) if layout == "Norm" else (nb, N, bs, dk)
    vshape = (nb, bs, N, dv) if layout == "Norm" else (nb, N, bs, dv)
    kc0, vc0 = rnd(*kshape), rnd(*vshape)
    print(f"[case] {layout} {dtype} T={T} N={N} dk={dk} dv={dv} nb={nb} bs={bs} slots={slot_dtype} "
          f"value={with_value} bad={bad_slots}", flush=True)
    kc, vc = kc0.to(gpu_device), vc0.to(gpu_device)
    sl = torch.from_numpy(slots).to(slot_dtype).to(gpu_device)
    if with_value:
        fb.fa_scatter_kv_cache(key.to(gpu_device), kc, sl, val.to(gpu_device), vc, layout=layout)
    else:
        fb.fa_scatter_kv_cache(key.to(gpu_device), kc, sl, layout=layout)
    torch.cuda.synchronize()
    ref_k, ref_v = kv_cache.scatter_kv_cache(bits(key), bits(kc0), slots, bits(val) if with_value else None,
                                             bits(vc0) if with_value else None, layout=layout)
    assert np.array_equal(bits(kc.cpu()), ref_k)
    if with_value:
        assert np.array_equal(bits(vc.cpu()), ref_v)
    else:
        assert torch.equal(vc.cpu(), vc0)


@pytest.mark.parametrize("layout", ["Norm", "NHSD"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16, torch.float32, torch.int8])
def test_scatter_small(gpu_device, layout, dtype):
    for i, (dk, dv, slot_dtype) in enumerate([(128, 128, torch.int32), (64, 40, torch.int64), (3, 5, torch.int32)]):
        _case(gpu_device, layout, dtype, T=37, N=3, dk=dk, dv=dv, nb=11, bs=16, slot_dtype=slot_dtype, seed=10 + i)
    _case(gpu_device, layout, dtype, T=20, N=2, dk=64, dv=64, nb=5, bs=8, slot_dtype=torch.int64, seed=20,
          bad_slots=5)
    _case(gpu_device, layout, dtype, T=9, N=4, dk=32, dv=32, nb=4, bs=4, slot_dtype=torch.int32, seed=21,
          with_value=False)


def test_scatter_empty(gpu_device):
    kc = torch.zeros(2, 4, 2, 8, dtype=torch.bfloat16, device=gpu_device)
    fb.fa_scatter_kv_cache(torch.zeros(0, 2, 8, dtype=torch.bfloat16, device=gpu_device), kc,
                           torch.zeros(0, dtype=torch.int32, device=gpu_device))
    torch.cuda.synchronize()
    assert torch.count_nonzero(kc) == 0


@pytest.mark.parametrize("layout", ["Norm", "NHSD"])
def test_scatter_prefill_size(gpu_device, layout):
    """A prefill chunk at serving size: 16384 tokens, 32 heads, D 128, bf16, every slot of a
    1024 x 16 cache written once."""
    _case(gpu_device, layout, torch.bfloat16, T=16384, N=32, dk=128, dv=128, nb=1024, bs=16,
          slot_dtype=torch.int64, seed=30)


@pytest.mark.parametrize("grid", [None, "1", "3"])
def test_scatter_segments_and_grid_stride(gpu_device, monkeypatch, grid):
    """Work units of 256 chunks: token counts of 1 and odd sizes, rows that end inside a unit,
    rows of several units (40 heads x D 128 = 1280 chunks), keys without values, padding slots;
    with the grid capped at 1 and 3 workgroups each one walks many units (the path huge
    inputs take)."""
    if grid is not None:
        monkeypatch.setenv("FA_SCATTER_GRID", grid)
    for i, T in enumerate((1, 3, 5, 38)):
        _case(gpu_device, "Norm", torch.bfloat16, T=T, N=3, dk=128, dv=64, nb=11, bs=16, slot_dtype=torch.int32,
              seed=40 + i, bad_slots=min(2, T - 1))
        _case(gpu_device, "NHSD", torch.float16, T=T, N=2, dk=24, dv=40, nb=7, bs=8, slot_dtype=torch.int64,
              seed=50 + i, with_value=(i % 2 == 0))
    _case(gpu_device, "Norm", torch.bfloat16, T=7, N=40, dk=128, dv=128, nb=4, bs=4, slot_dtype=torch.int64,
          seed=60, bad_slots=1)
    _case(gpu_device, "NHSD", torch.int8, T=6, N=5, dk=3, dv=7, nb=3, bs=4, slot_dtype=torch.int32, seed=61)
