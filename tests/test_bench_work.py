"""bench.py's per-family algorithmic work: every kernel family the library times inside a layer
step has a formula (none is silently zero), on every workload, training or not."""
from __future__ import annotations

import math
import os
import re

import pytest

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# families that never run inside a layer step (weight preparation, the router step)
NOT_IN_STEP = {"quant", "dequant", "router"}


def _families():
    src = open(os.path.join(ROOT, "grouped_nf4_gemm_amd", "csrc", "api.hip")).read()
    block = src[src.index("static const char *names[FAM_COUNT]"):]
    block = block[:block.index("};")]
    names = re.findall(r'"([a-z_0-9]+)"', block)
    assert "gemm_gate_up" in names and len(names) >= 10
    return [n for n in names if n not in NOT_IN_STEP]


@pytest.mark.parametrize("name", sorted(synth.WORKLOADS))
def test_every_step_family_has_work(name):
    s = synth.WORKLOADS[name]
    for fam in _families():
        for train in (False, True):
            fl, by = bench.step_work(s, fam, s.E, train)
            assert math.isfinite(fl) and math.isfinite(by) and by > 0, (name, fam, train)


def test_unknown_family_is_an_error():
    with pytest.raises(KeyError):
        bench.step_work(synth.WORKLOADS["tiny"], "no_such_kernel", 4, True)


def test_roof_picks_the_binding_roof():
    # a GEMM-like intensity is MFMA-bound, a copy is HBM-bound
    r = bench.roof_of(1e12, 1e9, 1.0)
    assert r["bound"] == "mfma" and abs(r["achieved"] - 1000.0) < 1e-6
    r = bench.roof_of(0.0, 8e9, 1.0)
    assert r["bound"] == "hbm" and abs(r["frac"] - 1.0) < 1e-9
