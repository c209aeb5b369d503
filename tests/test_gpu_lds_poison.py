"""LDS-poison debug build: the kernels with LDS tiles, compiled with FA_LDS_POISON, fill their
LDS with NaN bit patterns before the first load (fa_device.h). Outputs of that build must equal
the normal library's bit for bit and hold no NaN: then no kernel read a byte of LDS that none
of its loads or stores wrote (zero-filled tile rows past a sequence end, masked keys, the
mode-1 tile lists, the decode split buffers, the backward's LSE / Delta tiles). The cases run
in child processes, one per library, through tests/lds_poison_cases.py."""

import json
import os
import subprocess
import sys

import pytest

from masked_attention_forward_amd import build as fbuild

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def _run_cases(lib):
    env = dict(os.environ, FA_LIBRARY=lib)
    for k in ("FA_KERNEL", "FA_PERSIST", "FA_PS_SLOTS", "FA_DECODE", "FA_TABLE_ORDER"):
        env.pop(k, None)
    r = subprocess.run([sys.executable, os.path.join(HERE, "lds_poison_cases.py")], env=env, capture_output=True,
                       text=True, timeout=240)
    assert r.returncode == 0, f"{os.path.basename(lib)}: exit {r.returncode}\n{r.stderr[-3000:]}"
    return json.loads(r.stdout.strip().splitlines()[-1])


def test_lds_poison_build_matches_normal_build():
    if not os.path.exists(fbuild.LIBFA_POISON):
        pytest.fail("the LDS-poison library is not built (masked_attention_forward_amd/build.py builds it)")
    normal = _run_cases(fbuild.LIBFA)
    poison = _run_cases(fbuild.LIBFA_POISON)
    assert normal.keys() == poison.keys()
    nan_cases = sorted(c for c, r in normal.items() if r["nan"])
    assert not nan_cases, f"NaN in the normal build's outputs: {nan_cases}"
    diff = sorted(c for c in normal if normal[c] != poison[c])
    assert not diff, f"poisoned LDS changed the outputs of: {diff}"
