"""CPU oracle (test infrastructure only).

Python marshalling over liboracle.so, the plain C reference of the routed-expert
MoE layer with per-expert pre-activation LoRA over a 4-bit fused expert stack.
Only the tests, the smoke check and the benchmark's CPU-baseline leg import this
package; the HIP library never does, and this package imports nothing from it.

Parity pins live in tests/test_oracle_*.py.  Every function here is pinned
there against something other than itself (published values, closed forms,
brute force, finite differences, library routines).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "oracle.c")

FMT_NF4, FMT_NF4_DQ, FMT_MXFP4, FMT_INT8, FMT_FP8 = 0, 1, 2, 3, 4
_FMT = {"nf4": FMT_NF4, "nf4_dq": FMT_NF4_DQ, "mxfp4": FMT_MXFP4, "int8": FMT_INT8, "fp8": FMT_FP8}


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (plain C11 + OpenMP, no FMA contraction)."""
    if force or not os.path.exists(_SO):
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
               "-Wall", "-o", _SO, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
    return _SO


class _QW(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("E", ctypes.c_int32), ("N", ctypes.c_int32),
                ("K", ctypes.c_int32), ("codes", ctypes.c_void_p), ("scale", ctypes.c_void_p),
                ("scale2", ctypes.c_void_p), ("dq_table", ctypes.c_void_p), ("codebook", ctypes.c_void_p)]


class _Layer(ctypes.Structure):
    _fields_ = [("E", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("T", ctypes.c_int32), ("k", ctypes.c_int32),
                ("w_gu", ctypes.POINTER(_QW)), ("w_dn", ctypes.POINTER(_QW)),
                ("W1f", ctypes.c_void_p), ("W2f", ctypes.c_void_p),
                ("A1", ctypes.c_void_p), ("B1", ctypes.c_void_p), ("r1", ctypes.c_int32),
                ("s1", ctypes.c_double),
                ("A2", ctypes.c_void_p), ("B2", ctypes.c_void_p), ("r2", ctypes.c_int32),
                ("s2", ctypes.c_double),
                ("x", ctypes.c_void_p), ("ids", ctypes.c_void_p), ("topw", ctypes.c_void_p),
                ("post_act_delta", ctypes.c_int32), ("act", ctypes.c_int32), ("alpha", ctypes.c_double),
                ("limit", ctypes.c_double), ("b1", ctypes.c_void_p), ("b2", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        _lib = ctypes.CDLL(_SO)
        _lib.orc_moe_fwd.restype = ctypes.c_int32
        _lib.orc_moe_bwd.restype = ctypes.c_int32
        _lib.orc_version.restype = ctypes.c_int32
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def codebook() -> np.ndarray:
    out = np.zeros(16, np.float32)
    lib().orc_nf4_codebook(_p(out))
    return out


def bf16_round(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, np.float32)
    out = np.zeros(a.shape, np.uint16)
    lib().orc_bf16_round(_p(a), _p(out), ctypes.c_int64(a.size))
    return out


class QWeight:
    """A quantised stack [E, N, K] (K contiguous) in one of the three formats.  dq_table
    (fp32 [256], NF4_DQ) and codebook (fp32 [16], NF4 formats) replace the built-in code
    tables when given."""

    def __init__(self, fmt: str, E: int, N: int, K: int, codes, scale, scale2=None, dq_table=None,
                 codebook=None):
        self.fmt, self.E, self.N, self.K = fmt, E, N, K
        self.codes, self.scale, self.scale2 = codes, scale, scale2
        self.dq_table = None if dq_table is None else np.ascontiguousarray(dq_table, np.float32)
        self.codebook = None if codebook is None else np.ascontiguousarray(codebook, np.float32)
        assert self.dq_table is None or self.dq_table.shape == (256,)
        assert self.codebook is None or self.codebook.shape == (16,)

    def with_tables(self, dq_table=None, codebook=None) -> "QWeight":
        """The same bytes read through other code tables."""
        return QWeight(self.fmt, self.E, self.N, self.K, self.codes, self.scale, self.scale2,
                       dq_table, codebook)

    def struct(self) -> _QW:
        return _QW(_FMT[self.fmt], self.E, self.N, self.K, _p(self.codes), _p(self.scale),
                   _p(self.scale2), _p(self.dq_table), _p(self.codebook))


def quantize(fmt: str, w: np.ndarray) -> QWeight:
    """Quantise a stack [E, N, K] (fp32) along its contiguous last axis."""
    w = np.ascontiguousarray(w, np.float32)
    E, N, K = w.shape
    n = w.size
    if fmt in ("int8", "fp8"):  # one byte per element, an fp32 scale per 64
        codes = np.zeros(n, np.uint8)
        scale = np.zeros(n // 64, np.float32)
        (lib().orc_quant_int8 if fmt == "int8" else lib().orc_quant_fp8)(_p(w), ctypes.c_int64(n), _p(codes),
                                                                        _p(scale))
        return QWeight(fmt, E, N, K, codes, scale)
    codes = np.zeros(n // 2, np.uint8)
    if fmt == "nf4":
        scale = np.zeros(n // 64, np.float32)
        lib().orc_quant_nf4(_p(w), ctypes.c_int64(n), _p(codes), _p(scale))
        return QWeight(fmt, E, N, K, codes, scale)
    if fmt == "nf4_dq":
        scale = np.zeros(n // 64, np.uint8)
        scale2 = np.zeros((n // 64 + 255) // 256, np.float32)
        lib().orc_quant_nf4_dq(_p(w), ctypes.c_int64(n), _p(codes), _p(scale), _p(scale2))
        return QWeight(fmt, E, N, K, codes, scale, scale2)
    if fmt == "mxfp4":
        scale = np.zeros(n // 32, np.uint8)
        lib().orc_quant_mxfp4(_p(w), ctypes.c_int64(n), _p(codes), _p(scale))
        return QWeight(fmt, E, N, K, codes, scale)
    raise ValueError(fmt)


def e4m3_values() -> np.ndarray:
    """The value of each of the 256 FP8 E4M3 codes (NaN for 0x7F, 0xFF)."""
    lib().orc_e4m3_value.restype = ctypes.c_float
    return np.array([lib().orc_e4m3_value(ctypes.c_uint8(c)) for c in range(256)], np.float32)


def quantize_flat_nf4(w: np.ndarray):
    w = np.ascontiguousarray(w, np.float32).ravel()
    codes = np.zeros(w.size // 2, np.uint8)
    absmax = np.zeros(w.size // 64, np.float32)
    lib().orc_quant_nf4(_p(w), ctypes.c_int64(w.size), _p(codes), _p(absmax))
    return codes, absmax


def dequant(q: QWeight, want_f32: bool = True, want_bf16: bool = True):
    n = q.E * q.N * q.K
    f32 = np.zeros(n, np.float32) if want_f32 else None
    b16 = np.zeros(n, np.uint16) if want_bf16 else None
    lib().orc_dequant(ctypes.c_int32(_FMT[q.fmt]), ctypes.c_int64(n), _p(q.codes), _p(q.scale),
                      _p(q.scale2), _p(q.dq_table), _p(q.codebook), _p(f32), _p(b16))
    shp = (q.E, q.N, q.K)
    return (None if f32 is None else f32.reshape(shp)), (None if b16 is None else b16.reshape(shp))


def route(ids: np.ndarray, E: int):
    ids = np.ascontiguousarray(ids, np.int32)
    T, k = ids.shape
    M = T * k
    cnt = np.zeros(E + 1, np.int32)
    off = np.zeros(E + 1, np.int32)
    perm = np.zeros(max(M, 1), np.int32)[:M]
    inv = np.zeros(max(M, 1), np.int32)[:M]
    lib().orc_route(T, k, E, _p(ids), _p(cnt), _p(off), _p(perm), _p(inv))
    return cnt, off, perm, inv


def router_topk(logits: np.ndarray, k: int):
    """Top-k ids (larger logit first, ties to the lower id) and the softmax over them."""
    logits = np.ascontiguousarray(logits, np.float32)
    T, E = logits.shape
    ids = np.zeros((T, k), np.int32)
    w = np.zeros((T, k), np.float32)
    lib().orc_router_topk(T, E, k, _p(logits), _p(ids), _p(w))
    return ids, w


def router_bwd(w: np.ndarray, dw: np.ndarray, ids: np.ndarray, E: int) -> np.ndarray:
    """d logits [T, E] from d w [T, k] through the softmax over the chosen experts."""
    w = np.ascontiguousarray(w, np.float32)
    dw = np.ascontiguousarray(dw, np.float32)
    ids = np.ascontiguousarray(ids, np.int32)
    T, k = w.shape
    out = np.zeros((T, E), np.float32)
    lib().orc_router_bwd(T, E, k, _p(w), _p(dw), _p(ids), _p(out))
    return out


class Layer:
    """Arguments of one layer call, kept alive for the C side."""

    def __init__(self, E, H, I, T, k, x, ids, topw, w_gu=None, w_dn=None, W1f=None, W2f=None,
                 A1=None, B1=None, s1=0.0, A2=None, B2=None, s2=0.0, post_act_delta=False,
                 act=None):
        """act: None for the stock act(gate) * up, or a dict {alpha, limit, b1, b2} for the
        clamped GLU over interleaved gate/up rows (b1 bf16 [E, 2I], b2 bf16 [E, H], each
        nullable)."""
        self.keep = []

        def arr(a, dt):
            if a is None:
                return None
            a = np.ascontiguousarray(a, dt)
            self.keep.append(a)
            return a

        self.x = arr(x, np.uint16)
        self.ids = arr(ids, np.int32)
        self.topw = arr(topw, np.float32)
        self.W1f, self.W2f = arr(W1f, np.float32), arr(W2f, np.float32)
        self.A1, self.B1 = arr(A1, np.uint16), arr(B1, np.uint16)
        self.A2, self.B2 = arr(A2, np.uint16), arr(B2, np.uint16)
        self.r1 = 0 if A1 is None else self.A1.shape[1]
        self.r2 = 0 if A2 is None else self.A2.shape[1]
        a = act or {}
        self.b1, self.b2 = arr(a.get("b1"), np.uint16), arr(a.get("b2"), np.uint16)
        self.qgu = w_gu.struct() if w_gu is not None else None
        self.qdn = w_dn.struct() if w_dn is not None else None
        self.keep += [w_gu, w_dn]
        self.c = _Layer(E, H, I, T, k,
                        ctypes.pointer(self.qgu) if self.qgu else None,
                        ctypes.pointer(self.qdn) if self.qdn else None,
                        _p(self.W1f), _p(self.W2f), _p(self.A1), _p(self.B1), self.r1, float(s1),
                        _p(self.A2), _p(self.B2), self.r2, float(s2),
                        _p(self.x), _p(self.ids), _p(self.topw), int(post_act_delta),
                        1 if act else 0, float(a.get("alpha", 0.0)), float(a.get("limit", 0.0)),
                        _p(self.b1), _p(self.b2))
        self.E, self.H, self.I, self.T, self.k = E, H, I, T, k


def layer_from_inputs(inp, w_gu=None, w_dn=None, dense=False, lora=True, post_act_delta=False, act=None):
    s = inp.shape
    return Layer(s.E, s.H, s.I, s.T, s.k, inp.x, inp.ids, inp.topw,
                 w_gu=w_gu, w_dn=w_dn,
                 W1f=inp.W1 if dense else None, W2f=inp.W2 if dense else None,
                 A1=inp.A1 if lora else None, B1=inp.B1 if lora else None, s1=s.scaling,
                 A2=inp.A2 if lora else None, B2=inp.B2 if lora else None, s2=s.scaling,
                 post_act_delta=post_act_delta, act=act)


def _mask(L: Layer, tokens):
    if tokens is None:
        return None
    m = np.zeros(L.T, np.uint8)
    m[np.asarray(tokens, np.int64)] = 1
    L.keep.append(m)
    return m


def moe_fwd(L: Layer, tokens=None, want_O: bool = False):
    """y fp64 [T, H] (only the selected tokens are computed) and optionally O [T*k, H]."""
    y = np.zeros((L.T, L.H), np.float64)
    O = np.zeros((L.T * L.k, L.H), np.float64) if want_O else None
    m = _mask(L, tokens)
    rc = lib().orc_moe_fwd(ctypes.byref(L.c), _p(m), _p(y), _p(O))
    assert rc == 0
    return (y, O) if want_O else y


def moe_bwd(L: Layer, dy: np.ndarray, tokens=None):
    """Gradients of sum(dy * y): dx [T,H], dw [T,k], dA1, dB1, dA2, dB2 (fp64)."""
    dy = np.ascontiguousarray(dy, np.uint16)
    E, H, I = L.E, L.H, L.I
    out = {
        "dx": np.zeros((L.T, H)),
        "dw": np.zeros((L.T, L.k)),
        "dA1": np.zeros((E, L.r1, H)) if L.r1 else None,
        "dB1": np.zeros((E, 2 * I, L.r1)) if L.r1 else None,
        "dA2": np.zeros((E, L.r2, I)) if L.r2 else None,
        "dB2": np.zeros((E, H, L.r2)) if L.r2 else None,
    }
    m = _mask(L, tokens)
    rc = lib().orc_moe_bwd(ctypes.byref(L.c), _p(m), _p(dy), _p(out["dx"]), _p(out["dw"]),
                           _p(out["dA1"]), _p(out["dB1"]), _p(out["dA2"]), _p(out["dB2"]))
    assert rc == 0
    return out
