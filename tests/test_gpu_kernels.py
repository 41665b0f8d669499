"""GPU bit-exact checks: 4-bit decode, quantisers and routing metadata against the
oracle (integer and byte work must match exactly; the decoded fp32 and bf16
weights are fixed by the format's closed form)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from grouped_nf4_gemm_amd import QStack, route, router_bwd, router_topk
from tests.gpu_helpers import require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _weights(E, N, K, seed, scale=0.02):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((E, N, K)) * scale).astype(np.float32)
    w[0, 0, :64] = 0.0          # an all-zero block
    w[-1, -1, :32] *= 50.0      # a block with a large scale
    return w


@pytest.mark.parametrize("fmt", ["nf4", "nf4_dq", "mxfp4", "int8", "fp8"])
@pytest.mark.parametrize("E,N,K", [(2, 96, 128), (3, 64, 2880), (1, 8, 64 * 300)])
def test_dequant_bitexact(fmt, E, N, K):
    print(f"dequant {fmt} {E}x{N}x{K}", flush=True)
    w = _weights(E, N, K, seed=E * 7 + N)
    q = oracle.quantize(fmt, w)
    f_ref, b_ref = oracle.dequant(q)
    d = QStack.from_host(fmt, E, N, K, q.codes, q.scale, q.scale2)
    f32, b16 = d.dequant(-1)
    assert np.array_equal(f32.cpu().numpy().view(np.uint32), f_ref.reshape(E * N, K).view(np.uint32))
    assert np.array_equal(b16.view(torch.int16).cpu().numpy().view(np.uint16), b_ref.reshape(E * N, K))
    # one expert at a time
    f1, b1 = d.dequant(E - 1)
    assert np.array_equal(f1.cpu().numpy(), f_ref[E - 1])


@pytest.mark.parametrize("fmt", ["nf4", "nf4_dq", "mxfp4", "int8", "fp8"])
def test_dequant_every_code(fmt):
    """All 256 code bytes under a spread of block scales (FP8: every finite code)."""
    E, N, K = 1, 64, 512
    rng = np.random.default_rng(3)
    byte = fmt in ("int8", "fp8")
    codes = np.tile(np.arange(256, dtype=np.uint8), E * N * K // (1 if byte else 2) // 256)
    if fmt == "fp8":
        codes[(codes & 0x7F) == 0x7F] = 0  # the two NaN codes never occur in a stack
    if byte:
        q = oracle.QWeight(fmt, E, N, K, codes, rng.uniform(0, 0.1, E * N * K // 64).astype(np.float32))
    elif fmt == "nf4":
        scale = rng.uniform(0, 3, E * N * K // 64).astype(np.float32)
        q = oracle.QWeight(fmt, E, N, K, codes, scale)
    elif fmt == "nf4_dq":
        scale = rng.integers(0, 256, E * N * K // 64).astype(np.uint8)
        scale2 = rng.uniform(0.01, 2, (E * N * K // 64 + 255) // 256).astype(np.float32)
        q = oracle.QWeight(fmt, E, N, K, codes, scale, scale2)
    else:
        scale = rng.integers(90, 160, E * N * K // 32).astype(np.uint8)
        q = oracle.QWeight(fmt, E, N, K, codes, scale)
    f_ref, b_ref = oracle.dequant(q)
    d = QStack.from_host(fmt, E, N, K, q.codes, q.scale, q.scale2)
    f32, b16 = d.dequant(-1)
    assert np.array_equal(f32.cpu().numpy().view(np.uint32), f_ref.reshape(N, K).view(np.uint32))
    assert np.array_equal(b16.view(torch.int16).cpu().numpy().view(np.uint16), b_ref.reshape(N, K))


def _tables(seed):
    """A signed, non-linear 8-bit absmax code and a permuted 4-bit codebook."""
    c = np.arange(256, dtype=np.float64)
    dq = (np.sign(c - 127.5) * ((c - 127.5) / 128.0) ** 2).astype(np.float32)
    cb = oracle.codebook()[np.random.default_rng(seed).permutation(16)].copy()
    return dq, cb


@pytest.mark.parametrize("fmt", ["nf4", "nf4_dq"])
def test_dequant_stack_tables(fmt):
    """The stack's own code tables replace the built-in ones bit for bit: every code
    byte, a non-linear signed absmax code (NF4_DQ) and a permuted codebook."""
    E, N, K = 2, 64, 512
    rng = np.random.default_rng(8)
    codes = np.tile(np.arange(256, dtype=np.uint8), E * N * K // 2 // 256)
    dq, cb = _tables(9)
    if fmt == "nf4":
        q = oracle.QWeight(fmt, E, N, K, codes, rng.uniform(0, 3, E * N * K // 64).astype(np.float32),
                           codebook=cb)
    else:
        q = oracle.QWeight(fmt, E, N, K, codes, rng.integers(0, 256, E * N * K // 64).astype(np.uint8),
                           rng.uniform(0.01, 2, (E * N * K // 64 + 255) // 256).astype(np.float32),
                           dq_table=dq, codebook=cb)
    f_ref, b_ref = oracle.dequant(q)
    d = QStack.from_host(fmt, E, N, K, q.codes, q.scale, q.scale2, dq_table=q.dq_table, codebook=q.codebook)
    f32, b16 = d.dequant(-1)
    assert np.array_equal(f32.cpu().numpy().view(np.uint32), f_ref.reshape(E * N, K).view(np.uint32))
    assert np.array_equal(b16.view(torch.int16).cpu().numpy().view(np.uint16), b_ref.reshape(E * N, K))


@pytest.mark.parametrize("T", [24, 150])
def test_layer_stack_tables(T):
    """The layer over NF4_DQ stacks read through their own tables (few routed rows: the
    weight-streaming kernels; many: the large tiles) matches the oracle reading the same
    tables, and differs from the built-in reading."""
    from tests.gpu_helpers import Case, assert_close, bf16_to_np

    s = synth.custom(4, 192, 320, T, 2, 16, 32.0, "nf4_dq", name=f"tables-t{T}")
    inp = synth.make_inputs(s, seed=300 + T)
    dq, cb = _tables(10)
    case = Case(inp, dq_table=dq, codebook=cb)
    out = case.run()
    L = case.oracle_layer()
    y_ref = oracle.moe_fwd(L)
    g = oracle.moe_bwd(L, inp.dy)
    assert_close(bf16_to_np(out["y"]), y_ref, "y")
    assert_close(bf16_to_np(out["dx"]), g["dx"], "dx")
    assert_close(out["dA_gu"].cpu().numpy(), g["dA1"], "dA_gu")
    plain = Case(inp).run(dgrad=False)
    assert not torch.equal(plain["y"], out["y"])


@pytest.mark.parametrize("fmt", ["nf4", "nf4_dq", "mxfp4", "int8", "fp8"])
def test_quantize_bitexact(fmt):
    E, N, K = 3, 80, 2880
    w = _weights(E, N, K, seed=11)
    q = oracle.quantize(fmt, w)
    g = QStack.quantize(fmt, torch.from_numpy(w).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(g.codes.cpu().numpy(), q.codes)
    assert np.array_equal(g.scale.cpu().numpy(), q.scale)
    if fmt == "nf4_dq":
        assert np.array_equal(g.scale2.cpu().numpy(), q.scale2)


@pytest.mark.parametrize("T,k,E,bad", [(0, 2, 4, False), (1, 2, 8, False), (37, 3, 5, True),
                                       (4096, 8, 128, True), (16384, 2, 8, False), (300, 1, 1, False),
                                       (5000, 4, 1024, True)])
def test_route_bitexact(T, k, E, bad):
    rng = np.random.default_rng(T + E)
    ids = rng.integers(0, E, (T, k)).astype(np.int32)
    if bad and T > 3:
        ids[1, 0] = E
        ids[3, k - 1] = -5
    cnt, off, perm, inv = oracle.route(ids, E)
    g = route(torch.from_numpy(ids).cuda(), E)
    torch.cuda.synchronize()
    for name, ref, got in zip(["cnt", "off", "perm", "inv"], [cnt, off, perm, inv], g):
        assert np.array_equal(got.cpu().numpy(), ref), name


def test_route_skewed_loads():
    s = synth.WORKLOADS["many-small"]
    inp = synth.make_inputs(s, weights=False)
    cnt, off, perm, inv = oracle.route(inp.ids, s.E)
    g = route(torch.from_numpy(inp.ids).cuda(), s.E)
    for ref, got in zip([cnt, off, perm, inv], g):
        assert np.array_equal(got.cpu().numpy(), ref)


# ---------------------------------------------------------------- router

ROUTER_CASES = [
    # T, E, k, distinct logit levels (None: continuous)
    (37, 8, 2, None),
    (64, 8, 1, None),
    (16, 64, 64, None),        # k = E = one wave
    (9, 1024, 8, None),        # 16 logits per lane
    (50, 128, 8, 2),           # many ties
    (33, 257, 5, 3),           # E not a multiple of 64
]


@pytest.mark.parametrize("T,E,k,levels", ROUTER_CASES)
def test_router_parity(T, E, k, levels):
    """ids bit-exact against the oracle; weights and logit gradients to fp32 rounding."""
    print(f"router T={T} E={E} k={k} levels={levels}", flush=True)
    rng = np.random.default_rng(T * 1000 + E + k)
    l = rng.standard_normal((T, E)).astype(np.float32)
    if levels:
        l = (np.round(l * levels) / levels).astype(np.float32)
    ids_ref, w_ref = oracle.router_topk(l, k)
    ids, w = router_topk(torch.from_numpy(l).cuda(), k)
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    assert np.max(np.abs(w.cpu().numpy() - w_ref)) <= 2e-6
    dw = rng.standard_normal((T, k)).astype(np.float32)
    d_ref = oracle.router_bwd(w_ref, dw, ids_ref, E)
    d = router_bwd(torch.from_numpy(w_ref).cuda(), torch.from_numpy(dw).cuda(), torch.from_numpy(ids_ref).cuda(), E)
    torch.cuda.synchronize()
    dn = d.cpu().numpy()
    assert np.max(np.abs(dn - d_ref)) <= 1e-5 * max(1.0, np.abs(d_ref).max())
    mask = np.ones((T, E), bool)
    np.put_along_axis(mask, ids_ref.astype(np.int64), False, axis=1)
    assert np.all(dn[mask] == 0)


def test_router_matches_harness_routing():
    """The device router reproduces the routing the workloads are built with."""
    s = synth.WORKLOADS["many-small"]
    rng = np.random.default_rng(77)
    l = rng.standard_normal((256, s.E)).astype(np.float32)
    ids_h, w_h = synth.route(l, s.k)
    ids, w = router_topk(torch.from_numpy(l).cuda(), s.k)
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), ids_h)
    assert np.max(np.abs(w.cpu().numpy() - w_h)) <= 2e-6
