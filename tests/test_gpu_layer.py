"""GPU parity of the layer (forward, input gradient, LoRA weight gradients)
against the oracle, element by element, on shapes the oracle finishes in seconds
but that span several tiles and ragged tails, plus the exact special cases."""
import numpy as np
import pytest
import torch

import synth
from grouped_nf4_gemm_amd import MoELayer, get_stats, reset_stats
from tests.gpu_helpers import Case, assert_close, bf16_to_np, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _check_all(case: Case, out: dict, tokens=None):
    L = case.oracle_layer()
    y_ref = oracle_fwd = None
    import oracle

    y_ref = oracle.moe_fwd(L, tokens=tokens)
    g_ref = oracle.moe_bwd(L, case.inp.dy, tokens=tokens) if "dx" in out else None
    sel = slice(None) if tokens is None else np.asarray(tokens)
    assert_close(bf16_to_np(out["y"])[sel], y_ref[sel], "y")
    if g_ref is None:
        return
    assert_close(bf16_to_np(out["dx"])[sel], g_ref["dx"][sel], "dx")
    assert_close(out["dw"].cpu().numpy()[sel], g_ref["dw"][sel], "d_topw")
    if case.lora and "dA_gu" in out:
        for k_gpu, k_ref in [("dA_gu", "dA1"), ("dB_gu", "dB1"), ("dA_dn", "dA2"), ("dB_dn", "dB2")]:
            assert_close(out[k_gpu].cpu().numpy(), g_ref[k_ref], k_gpu)
    del oracle_fwd


SHAPES = [
    # name, E, H, I, T, k, r, alpha, fmt
    ("tiny", 4, 64, 128, 32, 2, 8, 16.0, "nf4"),
    ("ragged", 5, 192, 320, 77, 3, 16, 32.0, "nf4"),
    ("multi-tile", 3, 256, 448, 300, 2, 64, 128.0, "nf4"),
    ("dq", 4, 320, 192, 150, 2, 8, 16.0, "nf4_dq"),
    ("mxfp4", 6, 192, 192, 100, 4, 8, 16.0, "mxfp4"),
    ("one-expert", 1, 128, 128, 200, 1, 8, 16.0, "nf4"),
    ("rank128", 2, 128, 256, 40, 2, 128, 256.0, "nf4"),
    ("int8-few", 4, 192, 320, 20, 2, 16, 32.0, "int8"),
    ("int8", 5, 192, 320, 150, 3, 16, 32.0, "int8"),
    ("fp8-few", 4, 256, 192, 20, 2, 8, 16.0, "fp8"),
    ("fp8", 3, 256, 448, 300, 2, 64, 128.0, "fp8"),
    # one column tile and 3 row tiles, K = 8192 / 16384: the fp32-epilogue GEMMs split every
    # tile along K (down into 2 parts, gate_up dgrad into 4), summed by the last part
    ("k-split", 3, 256, 8192, 300, 2, 16, 32.0, "nf4"),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_layer_parity(shape):
    name, E, H, I, T, k, r, alpha, fmt = shape
    print(f"layer parity {shape}", flush=True)
    s = synth.custom(E, H, I, T, k, r, alpha, fmt, name=name)
    case = Case(synth.make_inputs(s, seed=100 + E + H + T))
    reset_stats()
    out = case.run()
    st = get_stats()
    assert st["gemm_gate_up"] >= 1 and st["gemm_down"] >= 1
    assert st["gemm_down_dgrad"] >= 1 and st["gemm_gate_up_dgrad"] >= 1 and st["wgrad"] >= 4
    assert st["fallbacks"] == 0
    _check_all(case, out)


def test_tiny_workload_both_B():
    """The tiny workload, once with random B and once with B = 0."""
    for zero_B in (False, True):
        inp = synth.make_inputs(synth.WORKLOADS["tiny"], zero_B=zero_B)
        case = Case(inp)
        _check_all(case, case.run())


def test_zero_B_equals_no_adapter_bitwise():
    """B = 0: the K-extension adds exact zeros, so the GPU output and input gradient
    equal the adapter-free call bit for bit; dA = 0 exactly, dB does not vanish."""
    inp = synth.make_inputs(synth.custom(4, 128, 192, 64, 2, 16, 32.0), seed=5, zero_B=True)
    a = Case(inp, lora=True).run()
    b = Case(inp, lora=False).run()
    assert torch.equal(a["y"].view(torch.int16), b["y"].view(torch.int16))
    assert torch.equal(a["dx"].view(torch.int16), b["dx"].view(torch.int16))
    assert torch.count_nonzero(a["dA_gu"]) == 0 and torch.count_nonzero(a["dA_dn"]) == 0
    assert torch.count_nonzero(a["dB_gu"]) > 0 and torch.count_nonzero(a["dB_dn"]) > 0


def test_no_adapter_parity():
    inp = synth.make_inputs(synth.custom(3, 128, 128, 50, 2, 8, 16.0), seed=9)
    case = Case(inp, lora=False)
    _check_all(case, case.run())


def test_deterministic_and_duplicate_rows():
    """Run twice -> identical bits; a token duplicated in the batch gets identical rows."""
    inp = synth.make_inputs(synth.custom(4, 128, 192, 40, 2, 8, 16.0), seed=13)
    inp.x[7] = inp.x[3]
    inp.ids[7] = inp.ids[3]
    inp.topw[7] = inp.topw[3]
    inp.dy[7] = inp.dy[3]
    case = Case(inp)
    a = case.run()
    b = case.run()
    for k in a:
        assert torch.equal(a[k].view(torch.int32) if a[k].dtype == torch.float32 else a[k].view(torch.int16),
                           b[k].view(torch.int32) if b[k].dtype == torch.float32 else b[k].view(torch.int16)), k
    assert torch.equal(a["y"][7].view(torch.int16), a["y"][3].view(torch.int16))
    assert torch.equal(a["dx"][7].view(torch.int16), a["dx"][3].view(torch.int16))


def test_split_weight_gradients():
    """Weight gradients of two heavily routed experts split four ways (fp32 partial sums added
    in split order) and of two rarely routed ones not split: oracle parity on every row, and
    the same bits on a second call."""
    inp = synth.make_inputs(synth.custom(4, 256, 256, 2048, 2, 16, 32.0), seed=21)
    inp.ids[:1800] = np.array([0, 1], dtype=inp.ids.dtype)
    case = Case(inp)
    a = case.run()
    _check_all(case, a)
    b = case.run()
    for k in ("dA_gu", "dB_gu", "dA_dn", "dB_dn"):
        assert torch.equal(a[k].view(torch.int32), b[k].view(torch.int32)), k


def test_empty_experts_and_skew():
    """All tokens on one expert of four: the other experts' LoRA grads are exactly 0."""
    inp = synth.make_inputs(synth.custom(4, 128, 128, 90, 2, 8, 16.0), seed=17)
    inp.ids[:, 0] = 2
    inp.ids[:, 1] = 2
    case = Case(inp)
    out = case.run()
    _check_all(case, out)
    for k in ("dA_gu", "dB_gu", "dA_dn", "dB_dn"):
        g = out[k].cpu().numpy()
        assert np.all(g[[0, 1, 3]] == 0)


def test_out_of_range_ids_dropped():
    inp = synth.make_inputs(synth.custom(4, 128, 128, 20, 2, 8, 16.0), seed=19)
    inp.ids[2, 1] = 9
    inp.ids[5, 0] = -1
    case = Case(inp)
    out = case.run()
    assert case.layer.dropped_rows() == 2
    _check_all(case, out)


def test_zero_tokens():
    inp = synth.make_inputs(synth.custom(4, 64, 64, 0, 2, 8, 16.0), seed=1)
    case = Case(inp)
    out = case.run()
    assert out["y"].shape == (0, 64) and out["dx"].shape == (0, 64)
    for k in ("dA_gu", "dB_gu", "dA_dn", "dB_dn"):
        assert torch.count_nonzero(out[k]) == 0


@pytest.mark.parametrize("fmt", ["nf4", "nf4_dq", "mxfp4"])
def test_decode_strip_sequence(fmt):
    """Few tokens spread over many experts with wide gate_up stacks: one workgroup per
    eight strips of every touched expert would not fit on the device at once (16 experts x
    17 workgroups), so each wave of the weight-streaming kernel runs a sequence of strips."""
    s = synth.custom(16, 128, 2112, 8, 2, 16, 32.0, fmt, name=f"decode-seq-{fmt}")
    inp = synth.make_inputs(s, seed=57)
    inp.ids[:, 0] = np.arange(8)
    inp.ids[:, 1] = np.arange(8, 16)
    case = Case(inp, train=False)
    print(f"strip sequence {fmt}", flush=True)
    reset_stats()
    out = case.run(dgrad=False)
    assert get_stats()["fallbacks"] == 0
    _check_all(case, out)


def test_decode_shape_ignores_stale_lds():
    """Few tokens per expert (the weight-streaming path): blocks past the K range must
    not read LDS that this call did not write.  A call whose staged activations are all
    +Inf runs first, then a call with one token per expert; its output must be finite
    and equal, bit for bit, to the same call after a clean one."""
    s = synth.custom(4, 192, 192, 4, 1, 8, 16.0, "nf4", name="decode-stale")
    clean = synth.make_inputs(s, seed=41)
    clean.ids[:, 0] = np.arange(4)
    poison = synth.make_inputs(s, seed=41)
    poison.ids[:, 0] = 0
    poison.x[:] = np.uint16(0x7F80)  # +Inf in every activation
    case_c = Case(clean, train=False)
    case_p = Case(poison, train=False)
    case_c.run(dgrad=False)
    ref = case_c.run(dgrad=False)["y"].clone()
    case_p.run(dgrad=False)
    got = case_c.run(dgrad=False)["y"]
    assert torch.isfinite(got.float()).all()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    _check_all(case_c, {"y": got})


EXPAND_SHAPES = [
    # name, E, H, I, T, k, r, alpha, fmt  (more than 256 routed rows: the large tiles)
    ("x-ragged", 5, 192, 320, 150, 3, 16, 32.0, "nf4"),
    ("x-dq", 4, 320, 192, 150, 2, 8, 16.0, "nf4_dq"),
    ("x-mxfp4", 6, 192, 192, 100, 4, 8, 16.0, "mxfp4"),
    ("x-multi-tile", 3, 256, 448, 300, 2, 64, 128.0, "nf4"),
    ("x-int8", 4, 192, 320, 150, 3, 16, 32.0, "int8"),
    ("x-fp8", 3, 256, 192, 150, 2, 8, 16.0, "fp8"),
]


@pytest.mark.parametrize("shape", EXPAND_SHAPES, ids=[s[0] for s in EXPAND_SHAPES])
def test_expanded_stacks_bitwise(shape):
    """Large-batch calls that stream bf16 copies of the stacks give every output and
    gradient bit for bit equal to the same calls decoding inside the GEMM tiles, and
    both match the oracle."""
    name, E, H, I, T, k, r, alpha, fmt = shape
    print(f"expanded stacks {shape}", flush=True)
    inp = synth.make_inputs(synth.custom(E, H, I, T, k, r, alpha, fmt, name=name), seed=200 + E + T)
    reset_stats()
    a = Case(inp, expand=True).run()
    assert get_stats()["expand"] == 2
    reset_stats()
    b = Case(inp, expand=False).run()
    assert get_stats()["expand"] == 0
    for key in a:
        va = a[key].view(torch.int32) if a[key].dtype == torch.float32 else a[key].view(torch.int16)
        vb = b[key].view(torch.int32) if b[key].dtype == torch.float32 else b[key].view(torch.int16)
        assert torch.equal(va, vb), key
    _check_all(Case(inp, expand=True), a)


@pytest.mark.parametrize("T", [1, 8, 40])
def test_decode_forward_graph_replay(T):
    """The few-token forward is graph-capturable: no host synchronisation and no memset nodes.
    A captured forward is replayed several times, with other eager work between the replays
    (a forward on different tokens into another buffer), and every replay equals the eager
    forward bit for bit."""
    s = synth.custom(6, 256, 384, T, 2, 16, 32.0, "nf4", name=f"graph-t{T}")
    case = Case(synth.make_inputs(s, seed=90 + T), train=False)
    other = synth.make_inputs(s, seed=190 + T)
    x2 = torch.from_numpy(other.x.view(np.int16)).view(torch.bfloat16).cuda()
    ids2 = torch.from_numpy(other.ids).cuda()
    w2 = torch.from_numpy(other.topw).cuda()
    print(f"graph replay T={T}", flush=True)
    y = torch.empty(T, s.H, dtype=torch.bfloat16, device="cuda")
    y2 = torch.empty_like(y)
    case.layer.forward(case.x, case.ids, case.topw, y)
    torch.cuda.synchronize()
    ref = y.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        case.layer.forward(case.x, case.ids, case.topw, y)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        case.layer.forward(case.x, case.ids, case.topw, y)
    for _ in range(3):
        y.zero_()
        case.layer.forward(x2, ids2, w2, y2)  # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16))
    del graph
    _check_all(case, {"y": ref})


def test_layer_rejects_bad_arguments():
    """Tensors of the wrong dtype, shape or device are refused before any launch: int64 ids
    (torch.topk's default) would be read as pairs of int32, and a short or fp32 x would be
    read past its end."""
    inp = synth.make_inputs(synth.custom(4, 64, 64, 16, 2, 8, 16.0), seed=3)
    case = Case(inp)
    lay = case.layer
    reset_stats()
    bad = [
        lambda: lay.forward(case.x, case.ids.long(), case.topw),
        lambda: lay.forward(case.x.float(), case.ids, case.topw),
        lambda: lay.forward(case.x[:8].contiguous(), case.ids, case.topw),
        lambda: lay.forward(case.x.cpu(), case.ids, case.topw),
        lambda: lay.forward(case.x, case.ids, case.topw.double()),
        lambda: lay.forward(case.x, case.ids, case.topw, y=torch.empty(8, 64, dtype=torch.bfloat16, device="cuda")),
        lambda: lay.dgrad(case.ids, case.topw, case.dy[:, :32].contiguous()),
        lambda: lay.wgrad(case.x.t().contiguous().t()),
    ]
    for f in bad:
        with pytest.raises(ValueError):
            f()
    assert get_stats()["launches_total"] == 0


def _glu_act(s, seed):
    """Clamped-GLU biases that put some gates above the limit and some ups beyond +-limit,
    the rest well inside: every clamp decision is far from the limit in both precisions."""
    rng = np.random.default_rng(seed)
    b1 = rng.normal(0, 0.05, (s.E, 2 * s.I)).astype(np.float32)
    cols = rng.integers(0, 4, s.I)  # 0: none, 1: gate above, 2: up above, 3: up below
    b1[:, 0::2][:, cols == 1] += 10.0
    b1[:, 1::2][:, cols == 2] += 10.0
    b1[:, 1::2][:, cols == 3] -= 10.0
    b2 = rng.normal(0, 0.05, (s.E, s.H)).astype(np.float32)
    return synth.to_bf16_bits(b1), synth.to_bf16_bits(b2), cols


@pytest.mark.parametrize("T", [24, 150], ids=["weight-streaming", "large-tiles"])
def test_clamped_glu_layer(T):
    """The gpt-oss expert epilogue (interleaved gate/up rows, per-expert biases, clamped GLU
    with alpha 1.702 and limit 7) over MXFP4 stacks: forward, input gradient and LoRA
    gradients against the oracle, with clamping active on both halves."""
    import oracle

    s = synth.custom(6, 192, 192, T, 4, 8, 16.0, "mxfp4", name=f"glu-t{T}")
    inp = synth.make_inputs(s, seed=700 + T)
    b1, b2, cols = _glu_act(s, 800 + T)
    dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    act = {"kind": "clamped_glu", "alpha": 1.702, "limit": 7.0, "b_gu": dev(b1), "b_dn": dev(b2)}
    case = Case(inp)
    lay = MoELayer(case.w_gu, case.w_dn, case.l_gu, case.l_dn, s.T, s.k, train=True, act=act)
    reset_stats()
    y = lay.forward(case.x, case.ids, case.topw)
    dx, dw = lay.dgrad(case.ids, case.topw, case.dy)
    gw = lay.wgrad(case.x)
    torch.cuda.synchronize()
    assert get_stats()["fallbacks"] == 0
    L = oracle.layer_from_inputs(inp, case.q1, case.q2, act=dict(alpha=1.702, limit=7.0, b1=b1, b2=b2))
    y_ref = oracle.moe_fwd(L)
    g = oracle.moe_bwd(L, inp.dy)
    assert_close(bf16_to_np(y), y_ref, "y")
    assert_close(bf16_to_np(dx), g["dx"], "dx")
    assert_close(dw.cpu().numpy(), g["dw"], "d_topw")
    for k_gpu, k_ref in [("dA_gu", "dA1"), ("dB_gu", "dB1"), ("dA_dn", "dA2"), ("dB_dn", "dB2")]:
        assert_close(gw[k_gpu].cpu().numpy(), g[k_ref], k_gpu)
    # the clamped halves really are clamped: their LoRA-B gradient rows vanish exactly
    dB = gw["dB_gu"].cpu().numpy()
    assert np.all(dB[:, 0::2][:, cols == 1] == 0) and np.all(dB[:, 1::2][:, cols >= 2] == 0)
    assert np.abs(dB[:, 0::2][:, cols == 0]).min(initial=1.0) >= 0 and np.abs(dB).max() > 0
