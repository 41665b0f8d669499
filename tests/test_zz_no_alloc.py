"""The allocation-free forward (e4b_moe_fwd_noalloc) against the workspace forward
(e4b_moe_fwd) through the C ABI: two calls in a row, the second with a smaller input, each
equal bit for bit to the workspace forward on the same inputs (the same kernels run over
the library's scratch array instead of the caller's workspace)."""
import numpy as np
import pytest
import torch

import synth
from grouped_nf4_gemm_amd import get_stats, reset_stats
from grouped_nf4_gemm_amd._lib import E4B_ERR_WORKSPACE, E4BError, NOALLOC_SCRATCH_BYTES
from tests.gpu_helpers import Case, assert_close, bf16_to_np, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _pair(E, H, I, T, k, seed):
    s = synth.custom(E, H, I, T, k, 16, 32.0, "nf4", name=f"noalloc-t{T}")
    case = Case(synth.make_inputs(s, seed=seed), train=False)
    assert case.layer.ws_bytes <= NOALLOC_SCRATCH_BYTES
    ref = case.layer.forward(case.x, case.ids, case.topw)
    y = torch.full_like(ref, float("nan"))
    case.layer.forward_noalloc(case.x, case.ids, case.topw, y)
    torch.cuda.synchronize()
    return case, ref, y


def test_noalloc_forward_two_calls():
    # a large-tile call (600 routed rows), then a smaller decode-shaped call (10 rows)
    for E, H, I, T, k, seed in [(4, 256, 512, 300, 2, 61), (8, 512, 1024, 5, 2, 62)]:
        print(f"noalloc forward E={E} H={H} I={I} T={T} k={k}", flush=True)
        case, ref, y = _pair(E, H, I, T, k, seed)
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16))
        import oracle

        assert_close(bf16_to_np(y), oracle.moe_fwd(case.oracle_layer()), "y")


def test_noalloc_rejects_what_it_cannot_serve():
    """A training forward, and a layer whose workspace exceeds the scratch array, are refused
    before any launch."""
    from grouped_nf4_gemm_amd import LoRA, MoELayer, QStack

    case = Case(synth.make_inputs(synth.custom(2, 128, 128, 8, 2, 16, 32.0, "nf4"), seed=63), train=True)
    y = torch.empty(8, 128, dtype=torch.bfloat16, device="cuda")
    reset_stats()
    with pytest.raises(E4BError):
        case.layer.forward_noalloc(case.x, case.ids, case.topw, y)  # flags carry E4B_TRAIN
    E, H, I, T, k, r = 2, 4096, 4096, 4096, 2, 16
    w_gu, w_dn = QStack.empty("nf4", E, 2 * I, H), QStack.empty("nf4", E, H, I)
    b = lambda *shape: torch.empty(*shape, dtype=torch.bfloat16, device="cuda")
    big = MoELayer(w_gu, w_dn, LoRA(b(E, r, H), b(E, 2 * I, r), 2.0), LoRA(b(E, r, I), b(E, H, r), 2.0), T, k,
                   train=False)
    assert big.ws_bytes > NOALLOC_SCRATCH_BYTES
    ids = torch.zeros(T, k, dtype=torch.int32, device="cuda")
    topw = torch.zeros(T, k, dtype=torch.float32, device="cuda")
    with pytest.raises(E4BError) as ei:
        big.forward_noalloc(b(T, H), ids, topw, b(T, H))
    assert ei.value.status == E4B_ERR_WORKSPACE
    assert get_stats()["launches_total"] == 0
