"""GPU parity at the full sizes of the named workloads, in the launch
configuration the benchmark times.  The GPU computes every token; the oracle
computes a stratified subset of at least 256 tokens that covers every expert with
routed rows (the count is in the test id), and the LoRA weight gradients are
compared with dy zeroed outside that subset (the oracle's reduction then runs over
exactly the same rows)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_helpers import Case, assert_close, bf16_to_np, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


_INPUTS = {}


def _inputs(name):
    if name not in _INPUTS:
        _INPUTS.clear()
        print(f"workload {name}: generating", flush=True)
        _INPUTS[name] = synth.make_inputs(synth.WORKLOADS[name])
    return _INPUTS[name]


def _run(name: str, n_tokens: int, backward: bool, expand=None):
    s = synth.WORKLOADS[name]
    inp = _inputs(name)
    toks = synth.stratified_tokens(inp.ids, s.E, n_tokens) if n_tokens < s.T else np.arange(s.T)
    touched = np.unique(inp.ids[(inp.ids >= 0) & (inp.ids < s.E)])
    assert np.array_equal(np.unique(inp.ids[toks]), touched), "the subset covers every expert with rows"
    mask = np.zeros(s.T, bool)
    mask[toks] = True
    dy_sub = inp.dy.copy()
    dy_sub[~mask] = 0
    print(f"workload {name}: quantising + uploading ({len(toks)} checked tokens)", flush=True)
    case = Case(inp, expand=expand)
    dyt = torch.from_numpy(dy_sub.view(np.int16)).view(torch.bfloat16).cuda()
    out = case.run(dgrad=backward, wgrad=backward, dy=dyt)
    print(f"workload {name}: oracle", flush=True)
    L = case.oracle_layer()
    y_ref = oracle.moe_fwd(L, tokens=toks)
    assert_close(bf16_to_np(out["y"])[toks], y_ref[toks], f"{name} y")
    if not backward:
        return
    g = oracle.moe_bwd(L, dy_sub, tokens=toks)
    dx = bf16_to_np(out["dx"])
    assert_close(dx[toks], g["dx"][toks], f"{name} dx")
    assert np.all(dx[~mask] == 0), "tokens with dy = 0 must get dx = 0"
    assert_close(out["dw"].cpu().numpy()[toks], g["dw"][toks], f"{name} d_topw")
    for k_gpu, k_ref in [("dA_gu", "dA1"), ("dB_gu", "dB1"), ("dA_dn", "dA2"), ("dB_dn", "dB2")]:
        assert_close(out[k_gpu].cpu().numpy(), g[k_ref], f"{name} {k_gpu}")


@pytest.mark.parametrize("name", ["decode-t1", "decode-t8", "decode-t64"])
def test_decode_forward(name):
    _run(name, 64, backward=False)  # every token (T <= 64)


@pytest.mark.parametrize("n", [256], ids=lambda n: f"{n}tok")
def test_many_small_experts(n):
    _run("many-small", n, backward=True)


@pytest.mark.parametrize("n", [256], ids=lambda n: f"{n}tok")
def test_mxfp4_experts(n):
    _run("mxfp4", n, backward=True)


@pytest.mark.parametrize("expand", [False, True], ids=["in-register-decode-256tok", "bf16-copies-256tok"])
def test_large_batch(expand):
    _run("large", 256, backward=True, expand=expand)
