"""Seeded synthetic inputs for the routed-expert MoE layer.

Shared by the tests, the benchmark and the smoke check: the oracle and the HIP
library both consume what this module returns.  It holds no arithmetic of the
expert layer itself: it draws tensors, encodes them to bf16 with torch's own
conversion, and runs the frozen router (top-k over logits, softmax over the k
selected logits) that produces the routing inputs of the layer.  Quantisation to
4-bit is done by each side on its own (the oracle's quantiser, or the library's).

Workloads (expert-layer shapes of the model families the pages measure, with
synthetic values in place of real weights):
  tiny        E=4   H=64   I=128   T=32     top-2  r=8  alpha=16  NF4
  decode-tN   E=8   H=4096 I=14336 T=1/8/64 top-2  r=16 alpha=32  NF4
  many-small  E=128 H=2048 I=768   T=4096   top-8  r=16 alpha=32  NF4, expert bias N(0,1)
  mxfp4       E=32  H=2880 I=2880  T=2048   top-4  r=8  alpha=16  MXFP4
  large       E=8   H=4096 I=14336 T=16384  top-2  r=64 alpha=128 NF4 + double-quantised absmax,
                                                                   expert bias N(0,0.5)
Distributions: x, dy ~ N(0,1) (bf16); logits ~ N(0,1) fp32 (+ per-expert bias);
W ~ N(0, 0.02) fp32; A ~ U(+-1/sqrt(fan_in)) bf16; B ~ N(0, 0.01) bf16 (or 0).
Seed = 1000 + workload index, one independent stream per tensor (per expert for W).
"""
from __future__ import annotations

import dataclasses

import numpy as np

FMT_NAMES = {"nf4": 0, "nf4_dq": 1, "mxfp4": 2, "int8": 3, "fp8": 4}


@dataclasses.dataclass(frozen=True)
class Shape:
    name: str
    index: int
    E: int
    H: int
    I: int
    T: int
    k: int
    r: int
    alpha: float
    fmt: str
    bias_std: float = 0.0

    @property
    def scaling(self) -> float:
        return self.alpha / self.r

    @property
    def M(self) -> int:
        return self.T * self.k


WORKLOADS = {
    "tiny": Shape("tiny", 1, 4, 64, 128, 32, 2, 8, 16.0, "nf4"),
    "decode-t1": Shape("decode-t1", 2, 8, 4096, 14336, 1, 2, 16, 32.0, "nf4"),
    "decode-t8": Shape("decode-t8", 2, 8, 4096, 14336, 8, 2, 16, 32.0, "nf4"),
    "decode-t64": Shape("decode-t64", 2, 8, 4096, 14336, 64, 2, 16, 32.0, "nf4"),
    "many-small": Shape("many-small", 3, 128, 2048, 768, 4096, 8, 16, 32.0, "nf4", 1.0),
    "mxfp4": Shape("mxfp4", 4, 32, 2880, 2880, 2048, 4, 8, 16.0, "mxfp4"),
    "large": Shape("large", 5, 8, 4096, 14336, 16384, 2, 64, 128.0, "nf4_dq", 0.5),
}

_STREAMS = ("x", "logits", "bias", "W1", "W2", "A1", "B1", "A2", "B2", "dy")


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (uint16), via torch's round-to-nearest-even cast."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    return (a.astype(np.uint32) << 16).view(np.float32)


def _seqs(seed: int) -> dict:
    ss = np.random.SeedSequence(seed)
    return dict(zip(_STREAMS, ss.spawn(len(_STREAMS))))


def _normal_stack(seq: np.random.SeedSequence, shape, std: float) -> np.ndarray:
    """N(0, std) fp32 stack [E, ...], one child stream per expert, filled in parallel."""
    from concurrent.futures import ThreadPoolExecutor

    out = np.empty(shape, np.float32)
    kids = seq.spawn(shape[0])

    def fill(e):
        g = np.random.Generator(np.random.PCG64(kids[e]))
        g.standard_normal(out=out[e], dtype=np.float32)
        out[e] *= np.float32(std)

    with ThreadPoolExecutor(max_workers=min(16, max(1, shape[0]))) as ex:
        list(ex.map(fill, range(shape[0])))
    return out


def route(logits: np.ndarray, k: int) -> tuple[np.ndarray, np.ndarray]:
    """Frozen router: top-k experts by logit (ties -> lower id), softmax over the k chosen."""
    order = np.argsort(-logits, axis=1, kind="stable")[:, :k].astype(np.int32)
    sel = np.take_along_axis(logits, order, axis=1).astype(np.float32)
    sel = sel - sel.max(axis=1, keepdims=True)
    ex = np.exp(sel, dtype=np.float32)
    w = (ex / ex.sum(axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)
    return np.ascontiguousarray(order), np.ascontiguousarray(w)


@dataclasses.dataclass
class LayerInputs:
    shape: Shape
    x: np.ndarray      # uint16 bf16 [T, H]
    ids: np.ndarray    # int32 [T, k]
    topw: np.ndarray   # float32 [T, k]
    W1: np.ndarray     # float32 [E, 2I, H] (unquantised)
    W2: np.ndarray     # float32 [E, H, I]
    A1: np.ndarray     # uint16 bf16 [E, r, H]
    B1: np.ndarray     # uint16 bf16 [E, 2I, r]
    A2: np.ndarray     # uint16 bf16 [E, r, I]
    B2: np.ndarray     # uint16 bf16 [E, H, r]
    dy: np.ndarray     # uint16 bf16 [T, H]


def make_inputs(shape: Shape, seed: int | None = None, zero_B: bool = False,
                weights: bool = True) -> LayerInputs:
    """Draw every tensor of one layer call.  weights=False skips W1/W2 (empty arrays)."""
    s = shape
    seqs = _seqs(1000 + s.index if seed is None else seed)
    g = {k: np.random.Generator(np.random.PCG64(v)) for k, v in seqs.items()}
    x = to_bf16_bits(g["x"].standard_normal((s.T, s.H), dtype=np.float32))
    logits = g["logits"].standard_normal((s.T, s.E), dtype=np.float32)
    if s.bias_std:
        logits = logits + (g["bias"].standard_normal(s.E, dtype=np.float32) * np.float32(s.bias_std))
    ids, topw = route(logits, s.k)
    if weights:
        W1 = _normal_stack(seqs["W1"], (s.E, 2 * s.I, s.H), 0.02)
        W2 = _normal_stack(seqs["W2"], (s.E, s.H, s.I), 0.02)
    else:
        W1 = np.zeros((0,), np.float32)
        W2 = np.zeros((0,), np.float32)
    a1 = 1.0 / np.sqrt(s.H)
    a2 = 1.0 / np.sqrt(s.I)
    A1 = to_bf16_bits(g["A1"].uniform(-a1, a1, (s.E, s.r, s.H)).astype(np.float32))
    A2 = to_bf16_bits(g["A2"].uniform(-a2, a2, (s.E, s.r, s.I)).astype(np.float32))
    if zero_B:
        B1 = np.zeros((s.E, 2 * s.I, s.r), np.uint16)
        B2 = np.zeros((s.E, s.H, s.r), np.uint16)
    else:
        B1 = to_bf16_bits(g["B1"].normal(0.0, 0.01, (s.E, 2 * s.I, s.r)).astype(np.float32))
        B2 = to_bf16_bits(g["B2"].normal(0.0, 0.01, (s.E, s.H, s.r)).astype(np.float32))
    dy = to_bf16_bits(g["dy"].standard_normal((s.T, s.H), dtype=np.float32))
    return LayerInputs(s, x, ids, topw, W1, W2, A1, B1, A2, B2, dy)


def custom(E: int, H: int, I: int, T: int, k: int, r: int, alpha: float, fmt: str = "nf4",
           bias_std: float = 0.0, name: str = "custom") -> Shape:
    return Shape(name, 0, E, H, I, T, k, r, alpha, fmt, bias_std)


def stratified_tokens(ids: np.ndarray, E: int, n: int, seed: int = 7) -> np.ndarray:
    """Token subset of about n tokens that covers every expert with at least one row."""
    T = ids.shape[0]
    rng = np.random.Generator(np.random.PCG64(seed))
    chosen: set[int] = set()
    for e in range(E):
        toks = np.nonzero((ids == e).any(axis=1))[0]
        if toks.size and not any((ids[t] == e).any() for t in chosen if t in toks):
            chosen.add(int(toks[rng.integers(toks.size)]))
    rest = rng.permutation(T)
    for t in rest:
        if len(chosen) >= n:
            break
        chosen.add(int(t))
    return np.array(sorted(chosen), dtype=np.int64)
