"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a published
construction, a closed form evaluated by a library routine, brute force on small
inputs, an exact special case, or finite differences.  A plausible mistake in the
oracle (a dropped LoRA term, a wrong scaling, a swapped gate/up half, a transposed
operand, a wrong nibble order) fails at least one of them.
"""
import os

import numpy as np
import pytest
import torch

import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- NF4 table

def test_codebook_matches_published_table(orc):
    lit = np.loadtxt(os.path.join(GOLD, "nf4_codebook.txt"), dtype=np.float64)
    assert np.array_equal(orc.codebook().astype(np.float64), lit.astype(np.float32).astype(np.float64))


def test_codebook_matches_quantile_construction(orc):
    """NF4 = normalised quantiles of N(0,1): 8 positive levels from an even split of
    [offset, 0.5], 7 negative ones, plus an exact zero (QLoRA paper, NF4 section)."""
    from scipy.stats import norm

    offset = 1.0 - 0.5 * (1.0 / 32 + 1.0 / 30)
    pos = norm.ppf(np.linspace(offset, 0.5, 9)[:-1])
    neg = -norm.ppf(np.linspace(offset, 0.5, 8)[:-1])
    v = np.sort(np.concatenate([pos, [0.0], neg]))
    v /= v.max()
    cb = orc.codebook().astype(np.float64)
    assert np.abs(cb - v).max() < 5e-7


def test_codebook_invariants(orc):
    cb = orc.codebook()
    assert np.all(np.diff(cb) > 0)
    assert cb[0] == -1.0 and cb[7] == 0.0 and cb[15] == 1.0
    assert (cb < 0).sum() == 7 and (cb > 0).sum() == 8


# ----------------------------------------------------------------------------- bf16

def test_bf16_rounding_matches_torch(orc):
    rng = np.random.default_rng(0)
    a = rng.standard_normal(100000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 100000)
    # exact ties: low 16 bits 0x8000 with even and odd kept bits
    hi = rng.integers(0, 0x7F7F, 2000).astype(np.uint32) | (rng.integers(0, 2, 2000).astype(np.uint32) << 15)
    ties = (hi << 16 | 0x8000).view(np.float32)  # finite values only: NaN payloads are not compared
    a = np.concatenate([a.astype(np.float32), ties, np.float32([0.0, -0.0, np.inf, -np.inf, 3.4e38, 1e-45])])
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(orc.bf16_round(a), ref)


# ----------------------------------------------------------------------------- NF4 quant/dequant

def _blocks(rng, nblk, scale=0.02):
    return (rng.standard_normal((1, nblk, 64)) * scale).astype(np.float32)


def test_nf4_roundtrip_exact_codes(orc):
    """A block holding +-a and every code value times a quantises back to those codes."""
    cb = orc.codebook()
    rng = np.random.default_rng(1)
    for a in rng.uniform(1e-4, 10.0, 50).astype(np.float32):
        idx = rng.integers(0, 16, 64)
        idx[0] = 15  # guarantees absmax == a
        w = (cb[idx] * a).astype(np.float32).reshape(1, 1, 64)
        q = orc.quantize("nf4", w)
        assert q.scale[0] == a
        hi, lo = q.codes >> 4, q.codes & 15
        got = np.stack([hi, lo], axis=1).ravel()
        assert np.array_equal(got, idx)


def test_nf4_quant_bruteforce(orc):
    rng = np.random.default_rng(2)
    w = _blocks(rng, 300)
    w[0, 5] = 0.0  # an all-zero block
    q = orc.quantize("nf4", w)
    cb = orc.codebook()
    blocks = w.reshape(-1, 64)
    amax = np.abs(blocks).max(axis=1)
    assert np.array_equal(q.scale, amax)
    for b in range(blocks.shape[0]):
        if amax[b] == 0:
            want = np.full(64, 7)
        else:
            v = (blocks[b] / amax[b]).astype(np.float32)
            want = np.argmin(np.abs(v[:, None] - cb[None, :]).astype(np.float32), axis=1)
        byte = q.codes[b * 32:(b + 1) * 32]
        got = np.stack([byte >> 4, byte & 15], axis=1).ravel()  # element 2j -> high nibble
        assert np.array_equal(got, want), b


def test_nf4_dequant_closed_form(orc):
    """w = fp32(code) * absmax in one fp32 multiply; bf16 by round-to-nearest-even."""
    rng = np.random.default_rng(3)
    E, N, K = 2, 8, 128
    codes = rng.integers(0, 256, E * N * K // 2).astype(np.uint8)
    absmax = rng.uniform(0, 1, E * N * K // 64).astype(np.float32)
    q = orc.QWeight("nf4", E, N, K, codes, absmax)
    f32, b16 = orc.dequant(q)
    cb = np.loadtxt(os.path.join(GOLD, "nf4_codebook.txt")).astype(np.float32)
    nib = np.stack([codes >> 4, codes & 15], axis=1).ravel()
    want = cb[nib] * np.repeat(absmax, 64)
    assert want.dtype == np.float32
    assert np.array_equal(f32.ravel().view(np.uint32), want.view(np.uint32))
    ref16 = torch.from_numpy(want).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b16.ravel(), ref16)


def test_nf4_dq_scheme(orc):
    rng = np.random.default_rng(4)
    w = (rng.standard_normal((3, 64, 192)) * 0.02).astype(np.float32)  # 576 blocks: 3 groups, ragged tail
    w[1, :4] *= 7.0
    q = orc.quantize("nf4_dq", w)
    codes_p, amax = orc.quantize_flat_nf4(w)
    assert np.array_equal(q.codes, codes_p)  # 4-bit codes use the undoubled absmax
    nb = amax.size
    groups = [amax[g * 256:(g + 1) * 256] for g in range((nb + 255) // 256)]
    assert np.array_equal(q.scale2, np.array([g.max() for g in groups], np.float32))
    s2 = np.repeat(q.scale2, 256)[:nb]
    rec = (q.scale.astype(np.float32) / np.float32(255.0)).astype(np.float32) * s2
    assert np.all(np.abs(rec - amax) <= s2 / 510.0 * (1 + 1e-6))
    f32, b16 = orc.dequant(q)
    cb = orc.codebook()
    nib = np.stack([q.codes >> 4, q.codes & 15], axis=1).ravel()
    want = cb[nib] * np.repeat(rec.astype(np.float32), 64)
    assert np.array_equal(f32.ravel().view(np.uint32), want.view(np.uint32))


def test_stack_code_tables_reduce_to_builtin(orc):
    """A stack may carry its own code tables.  Passing the built-in values explicitly
    changes no bit; a 4-bit codebook permuted by p, read through codes relabelled by the
    inverse of p, decodes to the same weights; an absmax table scaled by 2 (exact in
    fp32) doubles every weight exactly."""
    rng = np.random.default_rng(11)
    w = (rng.standard_normal((2, 32, 256)) * 0.02).astype(np.float32)
    q = orc.quantize("nf4_dq", w)
    base_f, base_b = orc.dequant(q)
    cb = np.loadtxt(os.path.join(GOLD, "nf4_codebook.txt")).astype(np.float32)
    lin = (np.arange(256, dtype=np.float32) / np.float32(255.0)).astype(np.float32)
    f, b = orc.dequant(q.with_tables(dq_table=lin, codebook=cb))
    assert np.array_equal(f.view(np.uint32), base_f.view(np.uint32))
    assert np.array_equal(b, base_b)
    perm = rng.permutation(16)
    inv = np.argsort(perm)  # perm[inv[c]] = c
    hi, lo = inv[q.codes >> 4], inv[q.codes & 15]
    relabelled = ((hi << 4) | lo).astype(np.uint8)
    qp = orc.QWeight("nf4_dq", q.E, q.N, q.K, relabelled, q.scale, q.scale2, codebook=cb[perm])
    f, _ = orc.dequant(qp)
    assert np.array_equal(f.view(np.uint32), base_f.view(np.uint32))
    f, _ = orc.dequant(q.with_tables(dq_table=(2 * lin).astype(np.float32)))
    assert np.array_equal(f, 2 * base_f)


def test_dq_table_reduces_to_plain_nf4(orc):
    """A double-quantised stack read through any absmax table equals the plain NF4 stack
    whose fp32 absmax of block b is fp32(table[c_b] * scale2[b / 256]): the table only
    changes how the absmax is rebuilt (here a signed, non-linear 8-bit code)."""
    rng = np.random.default_rng(12)
    w = (rng.standard_normal((1, 48, 640)) * 0.02).astype(np.float32)  # 480 blocks: 2 groups
    q = orc.quantize("nf4_dq", w)
    c = np.arange(256, dtype=np.float64)
    table = (np.sign(c - 127.5) * ((c - 127.5) / 128.0) ** 2).astype(np.float32)
    s2 = np.repeat(q.scale2, 256)[: q.scale.size]
    amax = (table[q.scale] * s2).astype(np.float32)
    plain = orc.QWeight("nf4", q.E, q.N, q.K, q.codes, amax)
    want_f, want_b = orc.dequant(plain)
    got_f, got_b = orc.dequant(q.with_tables(dq_table=table))
    assert np.array_equal(got_f.view(np.uint32), want_f.view(np.uint32))
    assert np.array_equal(got_b, want_b)
    assert np.any(got_f < 0) and not np.array_equal(got_f, orc.dequant(q)[0])


# ----------------------------------------------------------------------------- MXFP4

E2M1 = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)


def test_mxfp4_dequant_closed_form(orc):
    rng = np.random.default_rng(5)
    E, N, K = 1, 4, 256
    codes = rng.integers(0, 256, E * N * K // 2).astype(np.uint8)
    scales = rng.integers(100, 150, E * N * K // 32).astype(np.uint8)
    q = orc.QWeight("mxfp4", E, N, K, codes, scales)
    f32, _ = orc.dequant(q)
    nib = np.stack([codes & 15, codes >> 4], axis=1).ravel()  # element 2j -> low nibble
    mag = E2M1[nib & 7] * np.where(nib & 8, -1.0, 1.0).astype(np.float32)
    want = np.ldexp(mag, np.repeat(scales.astype(np.int32) - 127, 32)).astype(np.float32)
    assert np.array_equal(f32.ravel(), want)


def test_mxfp4_quant_bruteforce(orc):
    rng = np.random.default_rng(6)
    w = (rng.standard_normal((1, 40, 64)) * 0.02).astype(np.float32)
    w[0, 0, :32] = 0.0
    q = orc.quantize("mxfp4", w)
    blocks = w.reshape(-1, 32)
    for b, blk in enumerate(blocks):
        amax = np.abs(blk).max()
        if amax == 0:
            assert q.scale[b] == 0
            continue
        e = int(np.floor(np.log2(np.float64(amax)))) - 2
        assert q.scale[b] == e + 127
        v = np.abs(blk.astype(np.float64)) / 2.0 ** e
        d = np.abs(v[:, None] - E2M1[None, :].astype(np.float64))
        best = np.argmin(d, axis=1)
        # ties -> even code
        for i in range(32):
            cand = np.nonzero(d[i] == d[i].min())[0]
            if cand.size > 1:
                best[i] = cand[cand % 2 == 0][0]
        best = np.where(v >= 6.0, 7, best)
        sign = np.where((blk < 0) & (best != 0), 8, 0)
        want = best + sign
        byte = q.codes[b * 16:(b + 1) * 16]
        got = np.stack([byte & 15, byte >> 4], axis=1).ravel()
        assert np.array_equal(got, want), b


def test_mxfp4_roundtrip_representable(orc):
    rng = np.random.default_rng(7)
    for _ in range(20):
        e = int(rng.integers(-12, 4))
        idx = rng.integers(0, 16, 32)
        idx[3] = 7  # magnitude 6 sets the shared exponent to e
        mag = E2M1[idx & 7] * np.where(idx & 8, -1.0, 1.0)
        w = np.ldexp(mag, e).astype(np.float32).reshape(1, 1, 32)
        q = orc.quantize("mxfp4", w)
        f32, _ = orc.dequant(q)
        assert np.array_equal(f32.ravel(), w.ravel())


# ----------------------------------------------------------------------------- 8-bit bases

def test_e4m3_table_matches_torch(orc):
    """The 256 FP8 E4M3 code values against torch's float8_e4m3fn decoding."""
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(orc.e4m3_values(), ref, equal_nan=True)


def test_fp8_quant_matches_torch_rounding(orc):
    """Codes are torch's round-to-nearest-even float8_e4m3fn conversion of w / (absmax / 448)."""
    rng = np.random.default_rng(41)
    w = (rng.standard_normal((2, 16, 256)) * 0.02).astype(np.float32)
    w[0, 0, :64] = 0.0
    q = orc.quantize("fp8", w)
    blocks = w.reshape(-1, 64)
    s = (np.abs(blocks).max(axis=1) / np.float32(448.0)).astype(np.float32)
    assert np.array_equal(q.scale, s)
    t = np.where(s[:, None] > 0, blocks / np.where(s > 0, s, 1)[:, None], 0).astype(np.float32)
    want = torch.from_numpy(np.clip(t, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    want[want == 0x80] = 0  # -0 is stored as +0
    assert np.array_equal(q.codes.reshape(-1, 64), want)


def test_int8_quant_bruteforce(orc):
    rng = np.random.default_rng(42)
    w = (rng.standard_normal((2, 16, 256)) * 0.02).astype(np.float32)
    w[1, 3, 64:128] = 0.0
    q = orc.quantize("int8", w)
    blocks = w.reshape(-1, 64)
    s = (np.abs(blocks).max(axis=1) / np.float32(127.0)).astype(np.float32)
    assert np.array_equal(q.scale, s)
    t = np.where(s[:, None] > 0, blocks / np.where(s > 0, s, 1)[:, None], 0).astype(np.float32)
    want = np.clip(np.rint(t), -127, 127).astype(np.int8).view(np.uint8)
    assert np.array_equal(q.codes.reshape(-1, 64), want)


@pytest.mark.parametrize("fmt", ["int8", "fp8"])
def test_8bit_roundtrip_and_dequant(orc, fmt):
    """Values on the format's grid with a power-of-two scale come back exactly, and dequant is
    one fp32 multiply of the decoded code (torch's float8 decoding for FP8) by the scale."""
    rng = np.random.default_rng(43)
    scale = np.float32(2.0 ** -5)
    if fmt == "int8":
        k = rng.integers(-127, 128, (4, 64))
        k[:, 5] = 127
        grid = k.astype(np.float32)
    else:
        vals = orc.e4m3_values()
        codes = rng.integers(0, 256, (4, 64))
        codes[(codes == 0x7F) | (codes == 0xFF) | (codes == 0x80)] = 1
        codes[:, 5] = 0x7E  # 448 fixes the scale
        grid = vals[codes]
    w = (grid * scale).astype(np.float32).reshape(1, 4, 64)
    q = orc.quantize(fmt, w)
    assert np.all(q.scale == scale)
    f32, b16 = orc.dequant(q)
    assert np.array_equal(f32.ravel(), w.ravel())
    # dequant of arbitrary codes and scales
    codes = rng.integers(0, 256, 4 * 64).astype(np.uint8)
    if fmt == "fp8":
        codes[(codes & 0x7F) == 0x7F] = 3
    sc = rng.uniform(0.001, 0.1, 4).astype(np.float32)
    q = orc.QWeight(fmt, 1, 4, 64, codes, sc)
    f32, b16 = orc.dequant(q)
    dec = codes.view(np.int8).astype(np.float32) if fmt == "int8" else \
        torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).float().numpy()
    want = (dec * np.repeat(sc, 64)).astype(np.float32)
    assert np.array_equal(f32.ravel().view(np.uint32), want.view(np.uint32))
    ref16 = torch.from_numpy(want).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b16.ravel(), ref16)


# ----------------------------------------------------------------------------- routing

@pytest.mark.parametrize("T,k,E", [(0, 2, 4), (1, 2, 8), (37, 3, 5), (200, 8, 128), (64, 1, 1)])
def test_route_bruteforce(orc, T, k, E):
    rng = np.random.default_rng(T * 31 + E)
    ids = rng.integers(0, E, (T, k)).astype(np.int32)
    if T > 3:
        ids[2, 0] = E + 3  # out of range: dropped
        ids[3, -1] = -1
    cnt, off, perm, inv = orc.route(ids, E)
    flat = ids.ravel().tolist()
    valid = [f for f in range(T * k) if 0 <= flat[f] < E]
    order = sorted(valid, key=lambda f: flat[f])  # Python's sort is stable
    assert perm[:len(order)].tolist() == order
    assert np.all(perm[len(order):] == -1)
    assert cnt[:E].tolist() == [flat.count(e) for e in range(E)]
    assert cnt[E] == T * k - len(valid)
    assert off.tolist() == [0] + np.cumsum(cnt[:E]).tolist()
    for p, f in enumerate(order):
        assert inv[f] == p
    assert all(inv[f] == -1 for f in range(T * k) if f not in set(valid))


# ----------------------------------------------------------------------------- forward

def _small(E=3, H=64, I=64, T=12, k=2, r=4, alpha=8.0, fmt="nf4", seed=11, zero_B=False):
    s = synth.custom(E, H, I, T, k, r, alpha, fmt)
    return synth.make_inputs(s, seed=seed, zero_B=zero_B)


def _f64(bits):
    return synth.bf16_bits_to_f32(bits).astype(np.float64)


def _dense_reformulation(inp, W1, W2, lora=True):
    """All experts for all tokens with dense fp64 torch matmuls, then a one-hot combine."""
    s = inp.shape
    X = torch.from_numpy(_f64(inp.x))
    Y = torch.zeros(s.T, s.H, dtype=torch.float64)
    C = torch.zeros(s.T, s.E, dtype=torch.float64)
    for j in range(s.k):
        C[torch.arange(s.T), torch.from_numpy(inp.ids[:, j].astype(np.int64))] += torch.from_numpy(
            inp.topw[:, j].astype(np.float64))
    for e in range(s.E):
        w1 = torch.from_numpy(W1[e].astype(np.float64))
        w2 = torch.from_numpy(W2[e].astype(np.float64))
        G = X @ w1.T
        if lora:
            A1, B1 = torch.from_numpy(_f64(inp.A1[e])), torch.from_numpy(_f64(inp.B1[e]))
            G = G + s.scaling * (X @ A1.T) @ B1.T
        h = torch.nn.functional.silu(G[:, :s.I]) * G[:, s.I:]
        o = h @ w2.T
        if lora:
            A2, B2 = torch.from_numpy(_f64(inp.A2[e])), torch.from_numpy(_f64(inp.B2[e]))
            o = o + s.scaling * (h @ A2.T) @ B2.T
        Y += C[:, e:e + 1] * o
    return Y.numpy()


@pytest.mark.parametrize("fmt", ["nf4", "nf4_dq", "mxfp4", "int8", "fp8"])
def test_forward_matches_dense_onehot(orc, fmt):
    inp = _small(fmt=fmt)
    q1, q2 = orc.quantize(fmt, inp.W1), orc.quantize(fmt, inp.W2)
    y = orc.moe_fwd(orc.layer_from_inputs(inp, q1, q2))
    W1, _ = orc.dequant(q1, want_bf16=False)
    W2, _ = orc.dequant(q2, want_bf16=False)
    ref = _dense_reformulation(inp, W1, W2)
    assert np.abs(y - ref).max() <= 1e-12 * np.abs(ref).max()


def test_forward_textbook_swiglu(orc):
    """E=1, k=1, w=1, no adapter: y = W2 (silu(W_gate x) * (W_up x))."""
    s = synth.custom(1, 64, 128, 5, 1, 4, 8.0)
    inp = synth.make_inputs(s, seed=3)
    inp.topw[:] = 1.0
    y = orc.moe_fwd(orc.layer_from_inputs(inp, dense=True, lora=False))
    X = torch.from_numpy(_f64(inp.x))
    w1 = torch.from_numpy(inp.W1[0].astype(np.float64))
    w2 = torch.from_numpy(inp.W2[0].astype(np.float64))
    mlp = (torch.nn.functional.silu(X @ w1[:128].T) * (X @ w1[128:].T)) @ w2.T
    assert np.abs(y - mlp.numpy()).max() <= 1e-12 * np.abs(mlp.numpy()).max()


def test_zero_B_is_exactly_base(orc):
    """B zero-initialised: the delta starts at exactly zero (solution page, component table)."""
    inp = _small(zero_B=True)
    q1, q2 = orc.quantize("nf4", inp.W1), orc.quantize("nf4", inp.W2)
    y_lora = orc.moe_fwd(orc.layer_from_inputs(inp, q1, q2, lora=True))
    y_base = orc.moe_fwd(orc.layer_from_inputs(inp, q1, q2, lora=False))
    assert np.array_equal(y_lora, y_base)
    g_lora = orc.moe_bwd(orc.layer_from_inputs(inp, q1, q2, lora=True), inp.dy)
    g_base = orc.moe_bwd(orc.layer_from_inputs(inp, q1, q2, lora=False), inp.dy)
    assert np.array_equal(g_lora["dx"], g_base["dx"])
    assert np.all(g_lora["dA1"] == 0) and np.all(g_lora["dA2"] == 0)
    assert np.abs(g_lora["dB1"]).max() > 0 and np.abs(g_lora["dB2"]).max() > 0


def test_lora_merge_identity(orc):
    """act((W + s B A) x) == act(W x + s B (A x)): the adapter equals a merged weight."""
    inp = _small(T=9, r=8, alpha=16.0)
    rng = np.random.default_rng(9)
    inp.B1[:] = synth.to_bf16_bits(rng.normal(0, 0.1, inp.B1.shape).astype(np.float32))
    inp.B2[:] = synth.to_bf16_bits(rng.normal(0, 0.1, inp.B2.shape).astype(np.float32))
    s = inp.shape
    y = orc.moe_fwd(orc.layer_from_inputs(inp, dense=True))
    W1m = inp.W1.astype(np.float64) + s.scaling * np.einsum("enr,erh->enh", _f64(inp.B1), _f64(inp.A1))
    W2m = inp.W2.astype(np.float64) + s.scaling * np.einsum("enr,eri->eni", _f64(inp.B2), _f64(inp.A2))
    ref = _dense_reformulation(inp, W1m, W2m, lora=False)
    assert np.abs(y - ref).max() <= 1e-12 * np.abs(ref).max()


def test_pre_activation_delta_is_distinguishable(orc):
    """act(W x + B A x) is not act(W x) + d: a planted post-activation delta must fail the
    bf16 parity gate (max <= 2e-2 max|ref|, relative L1 <= 5e-3) on the tiny workload."""
    inp = synth.make_inputs(synth.WORKLOADS["tiny"])
    q1, q2 = orc.quantize("nf4", inp.W1), orc.quantize("nf4", inp.W2)
    good = orc.moe_fwd(orc.layer_from_inputs(inp, q1, q2))
    bad = orc.moe_fwd(orc.layer_from_inputs(inp, q1, q2, post_act_delta=True))
    rel_l1 = np.abs(bad - good).sum() / np.abs(good).sum()
    rel_max = np.abs(bad - good).max() / np.abs(good).max()
    assert rel_l1 > 5e-3 * 4 or rel_max > 2e-2 * 4


def test_combine_order_k2_is_bitwise(orc):
    inp = _small(k=2)
    q1, q2 = orc.quantize("nf4", inp.W1), orc.quantize("nf4", inp.W2)
    y = orc.moe_fwd(orc.layer_from_inputs(inp, q1, q2))
    inp.ids[:] = inp.ids[:, ::-1].copy()
    inp.topw[:] = inp.topw[:, ::-1].copy()
    y2 = orc.moe_fwd(orc.layer_from_inputs(inp, q1, q2))
    assert np.array_equal(y, y2)


def test_duplicate_and_invalid_ids(orc):
    inp = _small(E=3, k=2, T=6)
    inp.ids[0] = [1, 1]          # duplicate: two separate routed rows
    inp.ids[1] = [2, 7]          # out of range: row dropped
    q1, q2 = orc.quantize("nf4", inp.W1), orc.quantize("nf4", inp.W2)
    y, O = orc.moe_fwd(orc.layer_from_inputs(inp, q1, q2), want_O=True)
    assert np.allclose(y[0], (float(inp.topw[0, 0]) + float(inp.topw[0, 1])) * O[0], rtol=1e-12, atol=0)
    assert np.array_equal(O[0], O[1])
    assert np.array_equal(y[1], inp.topw[1, 0] * O[2])
    assert np.all(O[3] == 0)


def test_token_mask_selects_rows(orc):
    inp = _small(T=10)
    q1, q2 = orc.quantize("nf4", inp.W1), orc.quantize("nf4", inp.W2)
    L = orc.layer_from_inputs(inp, q1, q2)
    full = orc.moe_fwd(L)
    sub = orc.moe_fwd(L, tokens=[1, 4, 7])
    assert np.array_equal(sub[[1, 4, 7]], full[[1, 4, 7]])
    assert np.all(sub[[0, 2, 3, 5, 6, 8, 9]] == 0)


# ----------------------------------------------------------------------------- backward

def _loss(orc, inp, dy64, **kw):
    y = orc.moe_fwd(orc.layer_from_inputs(inp, dense=True, **kw))
    return float((y * dy64).sum())


def _bf16_neighbours(bits):
    up = synth.bf16_bits_to_f32(np.uint16(bits + 1))
    dn = synth.bf16_bits_to_f32(np.uint16(bits - 1))
    return np.uint16(bits + 1), np.uint16(bits - 1), float(up) - float(dn)


def test_backward_finite_differences(orc):
    """Central differences over one-ulp bf16 steps (x, A1, B1: nonlinear) and exact
    differences (top-k weight, B2, A2: the loss is linear in them)."""
    inp = _small(E=2, H=64, I=64, T=6, k=2, r=4, alpha=8.0, seed=21)
    rng = np.random.default_rng(21)
    inp.B1[:] = synth.to_bf16_bits(rng.normal(0, 0.2, inp.B1.shape).astype(np.float32))
    inp.B2[:] = synth.to_bf16_bits(rng.normal(0, 0.2, inp.B2.shape).astype(np.float32))
    inp.W1 *= 5.0  # stronger gate nonlinearity
    dy64 = _f64(inp.dy)
    g = orc.moe_bwd(orc.layer_from_inputs(inp, dense=True), inp.dy)

    def central(arr, idx):
        keep = arr[idx]
        up, dn, step = _bf16_neighbours(keep)
        arr[idx] = up
        lp = _loss(orc, inp, dy64)
        arr[idx] = dn
        lm = _loss(orc, inp, dy64)
        arr[idx] = keep
        return (lp - lm) / step

    scale = {k: np.abs(v).max() for k, v in g.items() if v is not None}
    for idx in [(0, 3), (4, 10), (5, 63)]:
        assert abs(central(inp.x, idx) - g["dx"][idx]) <= 2e-3 * scale["dx"]
    for idx in [(0, 1, 5), (1, 3, 60)]:
        assert abs(central(inp.A1, idx) - g["dA1"][idx]) <= 2e-3 * scale["dA1"]
    for idx in [(0, 7, 2), (1, 100, 0), (0, 70, 3)]:
        assert abs(central(inp.B1, idx) - g["dB1"][idx]) <= 2e-3 * scale["dB1"]
    # exact differences where the loss is linear
    base = _loss(orc, inp, dy64)
    for (t, j) in [(0, 0), (3, 1)]:
        keep = inp.topw[t, j]
        inp.topw[t, j] = keep + np.float32(0.25)
        d = (_loss(orc, inp, dy64) - base) / float(np.float32(keep + np.float32(0.25)) - keep)
        inp.topw[t, j] = keep
        assert abs(d - g["dw"][t, j]) <= 1e-9 * max(1.0, abs(d))
    for name, idxs in [("B2", [(0, 1, 2), (1, 5, 3)]), ("A2", [(0, 1, 2), (1, 3, 50)])]:
        arr = getattr(inp, name)
        for idx in idxs:
            keep = arr[idx]
            arr[idx] = synth.to_bf16_bits(np.float32([synth.bf16_bits_to_f32(keep) + 0.5]))[0]
            step = float(synth.bf16_bits_to_f32(arr[idx])) - float(synth.bf16_bits_to_f32(keep))
            d = (_loss(orc, inp, dy64) - base) / step
            arr[idx] = keep
            assert abs(d - g["d" + name][idx]) <= 1e-8 * max(1.0, np.abs(g["d" + name]).max())


def test_backward_adjoint_in_B2(orc):
    """The loss is linear in B2: L(V) - L(0) = <dL/dB2, V> for any V."""
    inp = _small(E=2, T=8, seed=5)
    dy64 = _f64(inp.dy)
    rng = np.random.default_rng(5)
    V = synth.to_bf16_bits(rng.normal(0, 0.3, inp.B2.shape).astype(np.float32))
    inp.B2[:] = 0
    l0 = _loss(orc, inp, dy64)
    g = orc.moe_bwd(orc.layer_from_inputs(inp, dense=True), inp.dy)
    inp.B2[:] = V
    l1 = _loss(orc, inp, dy64)
    lhs = l1 - l0
    rhs = float((g["dB2"] * _f64(V)).sum())
    assert abs(lhs - rhs) <= 1e-10 * abs(rhs)


def test_backward_mask_equals_zeroed_dy(orc):
    """Gradients of a token subset equal full gradients with dy zeroed elsewhere."""
    inp = _small(T=10, seed=8)
    q1, q2 = orc.quantize("nf4", inp.W1), orc.quantize("nf4", inp.W2)
    L = orc.layer_from_inputs(inp, q1, q2)
    toks = [0, 3, 9]
    dyz = inp.dy.copy()
    keep = np.zeros(10, bool)
    keep[toks] = True
    dyz[~keep] = 0
    a = orc.moe_bwd(L, dyz)
    b = orc.moe_bwd(L, inp.dy, tokens=toks)
    for k in ["dA1", "dB1", "dA2", "dB2"]:
        assert np.allclose(a[k], b[k], rtol=1e-12, atol=1e-300)
    assert np.array_equal(a["dx"][toks], b["dx"][toks])


# ---------------------------------------------------------------- router (top-k + softmax)

def _router_logits(T, E, seed, levels=None):
    rng = np.random.default_rng(seed)
    l = rng.standard_normal((T, E)).astype(np.float32)
    if levels:  # few distinct values: many ties
        l = np.round(l * levels) / levels
    return l.astype(np.float32)


@pytest.mark.parametrize("levels", [None, 2])
def test_router_ids_are_a_stable_descending_sort(orc, levels):
    """The chosen ids equal numpy's stable sort of the negated logits (ties: lower id first)."""
    for E, k in [(13, 1), (13, 4), (13, 13), (64, 8)]:
        l = _router_logits(40, E, 3 + E + k, levels)
        ids, _ = orc.router_topk(l, k)
        ref = np.argsort(-l, axis=1, kind="stable")[:, :k]
        assert np.array_equal(ids, ref), (E, k)


def test_router_weights_closed_form(orc):
    """Weights are exp(l - max) / sum over the chosen logits (float64 closed form)."""
    l = _router_logits(50, 32, 11)
    ids, w = orc.router_topk(l, 6)
    sel = np.take_along_axis(l.astype(np.float64), ids.astype(np.int64), axis=1)
    ex = np.exp(sel - sel.max(axis=1, keepdims=True))
    ref = ex / ex.sum(axis=1, keepdims=True)
    assert np.max(np.abs(w - ref)) < 1e-7
    assert np.max(np.abs(w.sum(axis=1) - 1.0)) < 1e-6
    assert np.all(np.diff(w, axis=1) <= 0)  # larger logit first


def test_router_k1_weight_is_one_and_matches_argmax(orc):
    l = _router_logits(30, 9, 5)
    ids, w = orc.router_topk(l, 1)
    assert np.array_equal(ids[:, 0], np.argmax(l, axis=1))
    assert np.all(w == 1.0)


def test_router_bwd_finite_differences(orc):
    """d logits from d w equals central finite differences (float64) of <dw, w(logits)> with
    the chosen ids held fixed; ids outside the top-k get zero."""
    T, E, k = 6, 10, 3
    l = _router_logits(T, E, 21).astype(np.float64)
    ids, w = orc.router_topk(l.astype(np.float32), k)
    dw = np.random.default_rng(4).standard_normal((T, k)).astype(np.float32)
    got = orc.router_bwd(w, dw, ids, E)

    def f(lt):
        sel = np.take_along_axis(lt, ids.astype(np.int64), axis=1)
        ex = np.exp(sel - sel.max(axis=1, keepdims=True))
        return np.sum(dw * ex / ex.sum(axis=1, keepdims=True))

    eps = 1e-6
    num = np.zeros_like(l)
    for t in range(T):
        for e in range(E):
            lp, lm = l.copy(), l.copy()
            lp[t, e] += eps
            lm[t, e] -= eps
            num[t, e] = (f(lp) - f(lm)) / (2 * eps)
    assert np.max(np.abs(got - num)) < 1e-5
    mask = np.ones((T, E), bool)
    np.put_along_axis(mask, ids.astype(np.int64), False, axis=1)
    assert np.all(got[mask] == 0)


# ----------------------------------------------------------------------------- clamped GLU (gpt-oss experts)

def _glu_case(seed, limit=1e30, alpha=2.0, gate_bias=0.0, up_bias=0.0, b2=True, T=10):
    inp = _small(E=3, H=64, I=64, T=T, k=2, r=4, alpha=8.0, seed=seed)
    rng = np.random.default_rng(seed + 1000)
    s = inp.shape
    b1 = rng.normal(0, 0.05, (s.E, 2 * s.I)).astype(np.float32)
    b1[:, 0::2] += np.float32(gate_bias)
    b1[:, 1::2] += np.float32(up_bias)
    act = dict(alpha=alpha, limit=limit, b1=synth.to_bf16_bits(b1),
               b2=synth.to_bf16_bits(rng.normal(0, 0.05, (s.E, s.H)).astype(np.float32)) if b2 else None)
    return inp, act


def test_clamped_glu_reduces_to_stock_swiglu(orc):
    """With the clamp out of reach, the clamped GLU over interleaved rows equals the stock
    SwiGLU layer after a change of variables: de-interleave the rows, carry the gate_up
    biases and the +1 on up in one extra constant input feature, and absorb alpha by scaling
    the gate rows by alpha and the up rows by 1/alpha (exact for alpha = 2).  Gradients map
    back by the same change of variables."""
    inp, act = _glu_case(31, b2=False)
    s = inp.shape
    E, H, I, a = s.E, s.H, s.I, act["alpha"]
    Lg = orc.layer_from_inputs(inp, dense=True, act=act)
    y_g = orc.moe_fwd(Lg)
    g_g = orc.moe_bwd(Lg, inp.dy)
    H2 = H + 1
    one = synth.to_bf16_bits(np.float32([1.0]))[0]
    x2 = np.zeros((s.T, H2), np.uint16)
    x2[:, :H] = inp.x
    x2[:, H] = one
    b1 = synth.bf16_bits_to_f32(act["b1"])
    W1 = inp.W1
    W1s = np.zeros((E, 2 * I, H2), np.float32)
    W1s[:, :I, :H] = a * W1[:, 0::2, :]
    W1s[:, I:, :H] = W1[:, 1::2, :] / np.float32(a)
    W1s[:, :I, H] = a * b1[:, 0::2]
    W1s[:, I:, H] = (b1[:, 1::2] + np.float32(1.0)) / np.float32(a)  # exact in fp32
    A1s = np.zeros((E, s.r, H2), np.uint16)
    A1s[:, :, :H] = inp.A1
    B1 = synth.bf16_bits_to_f32(inp.B1)
    B1s = synth.to_bf16_bits(np.concatenate([a * B1[:, 0::2, :], B1[:, 1::2, :] / np.float32(a)], axis=1))
    W2s = np.zeros((E, H2, I), np.float32)
    W2s[:, :H] = inp.W2
    B2s = np.zeros((E, H2, s.r), np.uint16)
    B2s[:, :H] = inp.B2
    Ls = orc.Layer(E, H2, I, s.T, s.k, x2, inp.ids, inp.topw, W1f=W1s, W2f=W2s, A1=A1s, B1=B1s,
                   s1=s.scaling, A2=inp.A2, B2=B2s, s2=s.scaling)
    y_s = orc.moe_fwd(Ls)
    assert np.allclose(y_s[:, :H], y_g, rtol=1e-9, atol=1e-12 * np.abs(y_g).max())
    assert np.all(y_s[:, H] == 0)
    dy2 = np.zeros((s.T, H2), np.uint16)
    dy2[:, :H] = inp.dy
    g_s = orc.moe_bwd(Ls, dy2)
    close = lambda u, v: np.allclose(u, v, rtol=1e-8, atol=1e-11 * np.abs(v).max())
    assert close(g_s["dx"][:, :H], g_g["dx"])
    assert close(g_s["dw"], g_g["dw"])
    assert close(g_s["dA1"][:, :, :H], g_g["dA1"])
    assert close(a * g_s["dB1"][:, :I], g_g["dB1"][:, 0::2])
    assert close(g_s["dB1"][:, I:] / a, g_g["dB1"][:, 1::2])
    assert close(g_s["dA2"], g_g["dA2"]) and close(g_s["dB2"][:, :H], g_g["dB2"])


def test_clamped_glu_clamp_out_of_reach_is_bitwise_unclamped(orc):
    inp, act = _glu_case(32, limit=1e30)
    L1 = orc.layer_from_inputs(inp, dense=True, act=act)
    L2 = orc.layer_from_inputs(inp, dense=True, act=dict(act, limit=40.0))
    assert np.array_equal(orc.moe_fwd(L1), orc.moe_fwd(L2))
    g1, g2 = orc.moe_bwd(L1, inp.dy), orc.moe_bwd(L2, inp.dy)
    for k in g1:
        assert np.array_equal(g1[k], g2[k]), k


@pytest.mark.parametrize("half", ["gate", "up"])
def test_clamped_glu_saturates(orc, half):
    """Pre-activations beyond the limit (a bias of 60 against a limit of 7): the output no
    longer depends on that half's weights (doubling them changes no bit) and its LoRA-B
    gradient rows are exactly zero."""
    inp, act = _glu_case(33, limit=7.0, gate_bias=60.0 if half == "gate" else 0.0,
                         up_bias=60.0 if half == "up" else 0.0)
    rows = slice(0, None, 2) if half == "gate" else slice(1, None, 2)
    L1 = orc.layer_from_inputs(inp, dense=True, act=act)
    y1 = orc.moe_fwd(L1)
    g1 = orc.moe_bwd(L1, inp.dy)
    assert np.all(g1["dB1"][:, rows] == 0) and np.abs(g1["dB1"]).max() > 0
    inp.W1[:, rows, :] *= 2.0
    y2 = orc.moe_fwd(orc.layer_from_inputs(inp, dense=True, act=act))
    assert np.array_equal(y1, y2)


def test_clamped_glu_down_bias_is_additive(orc):
    """The down bias adds sum_j w[t,j] * b2[ids[t,j]] to y."""
    inp, act = _glu_case(34)
    y_b = orc.moe_fwd(orc.layer_from_inputs(inp, dense=True, act=act))
    y_0 = orc.moe_fwd(orc.layer_from_inputs(inp, dense=True, act=dict(act, b2=None)))
    b2 = synth.bf16_bits_to_f32(act["b2"]).astype(np.float64)
    want = np.einsum("tj,tjh->th", inp.topw.astype(np.float64), b2[inp.ids])
    assert np.allclose(y_b - y_0, want, rtol=1e-12, atol=1e-15)


def test_clamped_glu_backward_finite_differences(orc):
    """Central one-ulp differences of the loss, with a limit that clamps part of the gates and
    ups (alpha = 1.702, limit 0.6)."""
    inp, act = _glu_case(35, limit=0.6, alpha=1.702, T=6)
    inp.W1 *= 5.0
    dy64 = _f64(inp.dy)
    g = orc.moe_bwd(orc.layer_from_inputs(inp, dense=True, act=act), inp.dy)

    def loss():
        return float((orc.moe_fwd(orc.layer_from_inputs(inp, dense=True, act=act)) * dy64).sum())

    def central(arr, idx):
        keep = arr[idx]
        up, dn, step = _bf16_neighbours(keep)
        arr[idx] = up
        lp = loss()
        arr[idx] = dn
        lm = loss()
        arr[idx] = keep
        return (lp - lm) / step

    scale = {k: np.abs(v).max() for k, v in g.items() if v is not None}
    for idx in [(0, 3), (4, 10), (5, 63)]:
        assert abs(central(inp.x, idx) - g["dx"][idx]) <= 2e-3 * scale["dx"]
    for idx in [(0, 1, 5), (1, 3, 60)]:
        assert abs(central(inp.A1, idx) - g["dA1"][idx]) <= 2e-3 * scale["dA1"]
    for idx in [(0, 6, 2), (1, 101, 0), (0, 71, 3)]:
        assert abs(central(inp.B1, idx) - g["dB1"][idx]) <= 2e-3 * scale["dB1"]
