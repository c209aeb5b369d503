"""The exp2-throughput calibration kernel that the forward's second roofline is measured
against: it must run the iteration it claims (its outputs sit at the fixed point of
x = 2^(-x), times 8 chains) and report the exponential count of its launch."""

import math

import pytest
import torch

from masked_attention_forward_amd import binding as fb

pytestmark = pytest.mark.gpu


def _fixed_point():
    # Root of x = 2^(-x) by Newton's method on f(x) = x - 2^(-x), in float64.
    x = 0.5
    for _ in range(50):
        x -= (x - 2.0 ** -x) / (1.0 + math.log(2.0) * 2.0 ** -x)
    return x


def test_exp2_rate_probe_values_and_count():
    x = _fixed_point()
    assert abs(x - 2.0 ** -x) < 1e-15
    out = torch.full((64 * 256,), float("nan"), dtype=torch.float32, device="cuda")
    n = fb.fa_exp2_rate_probe(out, 4)
    torch.cuda.synchronize()
    assert n == 64 * 256 * 4 * 128
    # 64 steps of a contraction with factor ln2 * x (about 0.44) from starts in [0.5, 1):
    # every chain sits at the fp32 fixed point, within a few ulp of exp2's rounding.
    err = (out.double() - 8 * x).abs().max().item()
    assert err < 4e-6, err
