"""Torch-facing wrapper: device tensors in, C-ABI calls out (marshalling only).

`QStack` holds a frozen 4-bit stack [E, N, K] on the device, `LoRA` a stacked
per-expert adapter, and `MoELayer` one routed-expert layer with its caller-owned
workspace.  Every step of the layer runs in libe4b's HIP kernels.
"""
from __future__ import annotations

import ctypes
import dataclasses

import torch

from . import _lib
from ._lib import FMT, E4B_EXPAND, E4B_NO_EXPAND, E4B_TRAIN, check


def _ptr(t: torch.Tensor | None) -> int | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("device tensor expected")
    if not t.is_contiguous():
        raise ValueError("contiguous tensor expected")
    return t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


@dataclasses.dataclass
class QStack:
    """Frozen 4-bit stack [E, N, K] (K contiguous) on the device."""
    fmt: str
    E: int
    N: int
    K: int
    codes: torch.Tensor          # uint8 [E*N*K/2]
    scale: torch.Tensor          # fp32 / uint8
    scale2: torch.Tensor | None  # fp32 (NF4_DQ)

    def c(self) -> _lib.QWeight:
        return _lib.QWeight(FMT[self.fmt], self.E, self.N, self.K, _ptr(self.codes), _ptr(self.scale),
                            _ptr(self.scale2))

    @staticmethod
    def empty(fmt: str, E: int, N: int, K: int, device="cuda") -> "QStack":
        n = E * N * K
        codes = torch.empty(n // 2, dtype=torch.uint8, device=device)
        if fmt == "nf4":
            scale, scale2 = torch.empty(n // 64, dtype=torch.float32, device=device), None
        elif fmt == "nf4_dq":
            scale = torch.empty(n // 64, dtype=torch.uint8, device=device)
            scale2 = torch.empty((n // 64 + 255) // 256, dtype=torch.float32, device=device)
        elif fmt == "mxfp4":
            scale, scale2 = torch.empty(n // 32, dtype=torch.uint8, device=device), None
        else:
            raise ValueError(fmt)
        return QStack(fmt, E, N, K, codes, scale, scale2)

    @staticmethod
    def from_host(fmt: str, E: int, N: int, K: int, codes, scale, scale2=None, device="cuda") -> "QStack":
        t = lambda a: None if a is None else torch.from_numpy(a).to(device)
        return QStack(fmt, E, N, K, t(codes), t(scale), t(scale2))

    @staticmethod
    def quantize(fmt: str, w: torch.Tensor) -> "QStack":
        """Quantise an fp32 device stack [E, N, K] with the library's kernels."""
        E, N, K = w.shape
        q = QStack.empty(fmt, E, N, K, device=w.device)
        check(_lib.lib().e4b_quantize(FMT[fmt], E, N, K, _ptr(w.contiguous()), _ptr(q.codes),
                                      _ptr(q.scale), _ptr(q.scale2), _stream()), "e4b_quantize")
        return q

    def dequant(self, expert: int = -1, f32: bool = True, bf16: bool = True):
        rows = self.N * (self.E if expert < 0 else 1)
        o32 = torch.empty(rows, self.K, dtype=torch.float32, device=self.codes.device) if f32 else None
        o16 = torch.empty(rows, self.K, dtype=torch.bfloat16, device=self.codes.device) if bf16 else None
        qc = self.c()
        check(_lib.lib().e4b_dequant(ctypes.byref(qc), expert, _ptr(o32), _ptr(o16), _stream()),
              "e4b_dequant")
        return o32, o16


@dataclasses.dataclass
class LoRA:
    """Stacked adapter: A bf16 [E, r, K], B bf16 [E, N, r], delta = scaling * B (A v)."""
    A: torch.Tensor
    B: torch.Tensor
    scaling: float

    @property
    def r(self) -> int:
        return self.A.shape[1]

    def c(self) -> _lib.Lora:
        return _lib.Lora(_ptr(self.A), _ptr(self.B), self.r, float(self.scaling))


def _lora_c(l: LoRA | None):
    return ctypes.byref(l.c()) if l is not None else None


def route(ids: torch.Tensor, E: int):
    """Routing metadata of ids [T, k]: cnt [E+1], off [E+1], perm [T*k], inv [T*k]."""
    T, k = ids.shape
    M = T * k
    dev = ids.device
    cnt = torch.empty(E + 1, dtype=torch.int32, device=dev)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(max(M, 1), dtype=torch.int32, device=dev)
    inv = torch.empty(max(M, 1), dtype=torch.int32, device=dev)
    d = _lib.Desc(E, 64, 64, T, k, 0)
    check(_lib.lib().e4b_moe_route(ctypes.byref(d), _ptr(ids.contiguous()), _ptr(cnt), _ptr(off),
                                   _ptr(perm), _ptr(inv), _stream()), "e4b_moe_route")
    return cnt, off, perm[:M], inv[:M]


def router_topk(logits: torch.Tensor, k: int):
    """Top-k expert ids [T, k] (larger logit first, ties to the lower id) and the softmax
    weights over them [T, k], from fp32 logits [T, E]."""
    logits = logits.contiguous()
    T, E = logits.shape
    ids = torch.empty(max(T, 1), k, dtype=torch.int32, device=logits.device)
    w = torch.empty(max(T, 1), k, dtype=torch.float32, device=logits.device)
    check(_lib.lib().e4b_router_topk(_ptr(logits), T, E, k, _ptr(ids), _ptr(w), _stream()), "e4b_router_topk")
    return ids[:T], w[:T]


def router_bwd(topw: torch.Tensor, d_topw: torch.Tensor, ids: torch.Tensor, E: int) -> torch.Tensor:
    """d logits [T, E] from d topw [T, k], the chosen ids held fixed."""
    T, k = topw.shape
    out = torch.empty(max(T, 1), E, dtype=torch.float32, device=topw.device)
    check(_lib.lib().e4b_router_bwd(_ptr(topw.contiguous()), _ptr(d_topw.contiguous()), _ptr(ids.contiguous()), T, E,
                                    k, _ptr(out), _stream()), "e4b_router_bwd")
    return out[:T]


class MoELayer:
    """One routed-expert layer: frozen stacks w_gu [E, 2I, H], w_dn [E, H, I] plus
    optional adapters on each.  Owns its workspace (caller-side allocation).
    expand: None lets the library choose between decoding the stacks inside the GEMM
    tiles and streaming bf16 copies of them (large batches); True / False force it."""

    def __init__(self, w_gu: QStack, w_dn: QStack, l_gu: LoRA | None, l_dn: LoRA | None,
                 T: int, topk: int, train: bool = True, expand: bool | None = None):
        self.w_gu, self.w_dn, self.l_gu, self.l_dn = w_gu, w_dn, l_gu, l_dn
        self.E, self.H, self.I = w_gu.E, w_gu.K, w_dn.K
        self.T, self.topk = T, topk
        self.flags = (E4B_TRAIN if train else 0) | (
            0 if expand is None else E4B_EXPAND if expand else E4B_NO_EXPAND)
        self.desc = _lib.Desc(self.E, self.H, self.I, T, topk, self.flags)
        n = ctypes.c_size_t()
        check(_lib.lib().e4b_moe_workspace_size(ctypes.byref(self.desc), _lora_c(l_gu), _lora_c(l_dn),
                                                ctypes.byref(n)), "e4b_moe_workspace_size")
        self.ws_bytes = n.value
        self.ws = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device=w_gu.codes.device)
        self._qgu, self._qdn = w_gu.c(), w_dn.c()
        self._lgu = l_gu.c() if l_gu is not None else None
        self._ldn = l_dn.c() if l_dn is not None else None

    def _l(self, x):
        return ctypes.byref(x) if x is not None else None

    def forward(self, x, ids, topw, y=None):
        if y is None:
            y = torch.empty(self.T, self.H, dtype=torch.bfloat16, device=x.device)
        check(_lib.lib().e4b_moe_fwd(ctypes.byref(self.desc), ctypes.byref(self._qgu),
                                     ctypes.byref(self._qdn), self._l(self._lgu), self._l(self._ldn),
                                     _ptr(x), _ptr(ids), _ptr(topw), _ptr(y), _ptr(self.ws),
                                     self.ws_bytes, _stream()), "e4b_moe_fwd")
        return y

    def dgrad(self, ids, topw, dy, dx=None, d_topw=None, want_d_topw=True):
        if dx is None:
            dx = torch.empty(self.T, self.H, dtype=torch.bfloat16, device=dy.device)
        if d_topw is None and want_d_topw:
            d_topw = torch.empty(self.T, self.topk, dtype=torch.float32, device=dy.device)
        check(_lib.lib().e4b_moe_dgrad(ctypes.byref(self.desc), ctypes.byref(self._qgu),
                                       ctypes.byref(self._qdn), self._l(self._lgu), self._l(self._ldn),
                                       _ptr(ids), _ptr(topw), _ptr(dy), _ptr(dx), _ptr(d_topw),
                                       _ptr(self.ws), self.ws_bytes, _stream()), "e4b_moe_dgrad")
        return dx, d_topw

    def wgrad(self, x, out=None):
        dev = x.device
        E, H, I = self.E, self.H, self.I
        if out is None:
            out = {}
            if self.l_gu is not None:
                r = self.l_gu.r
                out["dA_gu"] = torch.empty(E, r, H, dtype=torch.float32, device=dev)
                out["dB_gu"] = torch.empty(E, 2 * I, r, dtype=torch.float32, device=dev)
            if self.l_dn is not None:
                r = self.l_dn.r
                out["dA_dn"] = torch.empty(E, r, I, dtype=torch.float32, device=dev)
                out["dB_dn"] = torch.empty(E, H, r, dtype=torch.float32, device=dev)
        check(_lib.lib().e4b_lora_wgrad(ctypes.byref(self.desc), self._l(self._lgu), self._l(self._ldn),
                                        _ptr(x), _ptr(self.ws), self.ws_bytes, _ptr(out.get("dA_gu")),
                                        _ptr(out.get("dB_gu")), _ptr(out.get("dA_dn")),
                                        _ptr(out.get("dB_dn")), _stream()), "e4b_lora_wgrad")
        return out

    def dropped_rows(self) -> int:
        v = ctypes.c_int32()
        check(_lib.lib().e4b_moe_check(ctypes.byref(self.desc), _ptr(self.ws), _stream(),
                                       ctypes.byref(v)), "e4b_moe_check")
        return v.value
