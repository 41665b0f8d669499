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
from ._lib import FMT, E4B_EXPAND, E4B_SEPARATE, E4B_TRAIN, check


def _ptr(t: torch.Tensor | None) -> int | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("device tensor expected")
    if not t.is_contiguous():
        raise ValueError("contiguous tensor expected")
    return t.data_ptr()


def _arg(t, name: str, dtype: torch.dtype, shape: tuple, device: torch.device) -> torch.Tensor:
    """Check one tensor argument before its pointer goes to the library: a wrong dtype,
    shape or device would make the kernels read or write outside the allocation."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: tensor expected")
    if t.dtype != dtype:
        raise ValueError(f"{name}: {dtype} expected, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(shape)} expected, got {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name}: tensor on {device} expected, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: contiguous tensor expected")
    return t


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


@dataclasses.dataclass
class QStack:
    """Frozen 4-bit stack [E, N, K] (K contiguous) on the device."""
    fmt: str
    E: int
    N: int
    K: int
    codes: torch.Tensor          # uint8 [E*N*K/2] (4-bit) or [E*N*K] (int8, fp8)
    scale: torch.Tensor          # fp32 (nf4, int8, fp8) / uint8 (nf4_dq absmax codes, mxfp4 E8M0)
    scale2: torch.Tensor | None  # fp32 (NF4_DQ)
    dq_table: torch.Tensor | None = None  # fp32 [256] (NF4_DQ; None = built-in c / 255)
    codebook: torch.Tensor | None = None  # fp32 [16] (NF4 formats; None = built-in NF4 table)

    def c(self) -> _lib.QWeight:
        for name, t, n in (("dq_table", self.dq_table, 256), ("codebook", self.codebook, 16)):
            if t is not None and (t.dtype != torch.float32 or t.numel() != n):
                raise ValueError(f"{name}: float32 tensor of {n} values expected")
        return _lib.QWeight(FMT[self.fmt], self.E, self.N, self.K, _ptr(self.codes), _ptr(self.scale),
                            _ptr(self.scale2), _ptr(self.dq_table), _ptr(self.codebook))

    @staticmethod
    def empty(fmt: str, E: int, N: int, K: int, device="cuda") -> "QStack":
        n = E * N * K
        codes = torch.empty(n if fmt in ("int8", "fp8") else n // 2, dtype=torch.uint8, device=device)
        if fmt in ("nf4", "int8", "fp8"):
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
    def from_host(fmt: str, E: int, N: int, K: int, codes, scale, scale2=None, device="cuda",
                  dq_table=None, codebook=None) -> "QStack":
        t = lambda a: None if a is None else torch.from_numpy(a).to(device)
        return QStack(fmt, E, N, K, t(codes), t(scale), t(scale2), t(dq_table), t(codebook))

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
    _arg(ids, "ids", torch.int32, (T, k), dev)
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
    T, E = logits.shape
    _arg(logits, "logits", torch.float32, (T, E), logits.device)
    ids = torch.empty(max(T, 1), k, dtype=torch.int32, device=logits.device)
    w = torch.empty(max(T, 1), k, dtype=torch.float32, device=logits.device)
    check(_lib.lib().e4b_router_topk(_ptr(logits), T, E, k, _ptr(ids), _ptr(w), _stream()), "e4b_router_topk")
    return ids[:T], w[:T]


def router_bwd(topw: torch.Tensor, d_topw: torch.Tensor, ids: torch.Tensor, E: int) -> torch.Tensor:
    """d logits [T, E] from d topw [T, k], the chosen ids held fixed."""
    T, k = topw.shape
    dev = topw.device
    _arg(topw, "topw", torch.float32, (T, k), dev)
    _arg(d_topw, "d_topw", torch.float32, (T, k), dev)
    _arg(ids, "ids", torch.int32, (T, k), dev)
    out = torch.empty(max(T, 1), E, dtype=torch.float32, device=dev)
    check(_lib.lib().e4b_router_bwd(_ptr(topw), _ptr(d_topw), _ptr(ids), T, E, k, _ptr(out), _stream()),
          "e4b_router_bwd")
    return out[:T]


class MoELayer:
    """One routed-expert layer: frozen stacks w_gu [E, 2I, H], w_dn [E, H, I] plus
    optional adapters on each.  Owns its workspace (caller-side allocation).
    expand=True asks the forward of a large batch to stream bf16 copies of the stacks
    (written into the workspace) instead of decoding them inside the GEMM tiles.
    separate=True runs a decode-shaped inference forward (at most 256 routed rows) as six
    launches instead of the default two."""

    def __init__(self, w_gu: QStack, w_dn: QStack, l_gu: LoRA | None, l_dn: LoRA | None,
                 T: int, topk: int, train: bool = True, expand: bool | None = None, act: dict | None = None,
                 separate: bool = False):
        """act: None for the stock act(gate) * up, or {"kind": "clamped_glu", "alpha": a,
        "limit": L, "b_gu": bf16 [E, 2I] or None, "b_dn": bf16 [E, H] or None} for the clamped
        GLU over interleaved gate/up rows (gpt-oss experts)."""
        self.w_gu, self.w_dn, self.l_gu, self.l_dn = w_gu, w_dn, l_gu, l_dn
        self.E, self.H, self.I = w_gu.E, w_gu.K, w_dn.K
        dev = w_gu.codes.device
        E, H, I = self.E, self.H, self.I
        for name, q, N, K in (("w_gu", w_gu, 2 * I, H), ("w_dn", w_dn, H, I)):
            if (q.E, q.N, q.K) != (E, N, K):
                raise ValueError(f"{name}: stack [{E}, {N}, {K}] expected, got [{q.E}, {q.N}, {q.K}]")
            n = E * N * K
            byte = q.fmt in ("int8", "fp8")
            _arg(q.codes, f"{name}.codes", torch.uint8, (n if byte else n // 2,), dev)
            nscale = n // 32 if q.fmt == "mxfp4" else n // 64
            _arg(q.scale, f"{name}.scale", torch.float32 if q.fmt in ("nf4", "int8", "fp8") else torch.uint8,
                 (nscale,), dev)
            if q.fmt == "nf4_dq":
                _arg(q.scale2, f"{name}.scale2", torch.float32, ((n // 64 + 255) // 256,), dev)
        for name, l, N, K in (("l_gu", l_gu, 2 * I, H), ("l_dn", l_dn, H, I)):
            if l is not None:
                _arg(l.A, f"{name}.A", torch.bfloat16, (E, l.r, K), dev)
                _arg(l.B, f"{name}.B", torch.bfloat16, (E, N, l.r), dev)
        self.T, self.topk = T, topk
        self.flags = (E4B_TRAIN if train else 0) | (E4B_EXPAND if expand else 0) | (E4B_SEPARATE if separate else 0)
        self._act = None
        if act is not None:
            b_gu, b_dn = act.get("b_gu"), act.get("b_dn")
            if b_gu is not None:
                _arg(b_gu, "b_gu", torch.bfloat16, (E, 2 * I), dev)
            if b_dn is not None:
                _arg(b_dn, "b_dn", torch.bfloat16, (E, H), dev)
            self._act_tensors = (b_gu, b_dn)
            self._act = _lib.Act(_lib.ACT[act.get("kind", "clamped_glu")], float(act.get("alpha", 1.702)),
                                 float(act.get("limit", 7.0)), _ptr(b_gu), _ptr(b_dn))
        self.desc = _lib.Desc(self.E, self.H, self.I, T, topk, self.flags,
                              ctypes.pointer(self._act) if self._act is not None else None)
        n = ctypes.c_size_t()
        check(_lib.lib().e4b_moe_workspace_size(ctypes.byref(self.desc), _lora_c(l_gu), _lora_c(l_dn),
                                                ctypes.byref(n)), "e4b_moe_workspace_size")
        self.ws_bytes = n.value
        self.device = w_gu.codes.device
        self.ws = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device=self.device)
        self._qgu, self._qdn = w_gu.c(), w_dn.c()
        self._lgu = l_gu.c() if l_gu is not None else None
        self._ldn = l_dn.c() if l_dn is not None else None

    def _l(self, x):
        return ctypes.byref(x) if x is not None else None

    def _routing(self, ids, topw):
        _arg(ids, "ids", torch.int32, (self.T, self.topk), self.device)
        _arg(topw, "topw", torch.float32, (self.T, self.topk), self.device)

    def forward(self, x, ids, topw, y=None):
        rows = (self.T, self.H)
        _arg(x, "x", torch.bfloat16, rows, self.device)
        self._routing(ids, topw)
        if y is None:
            y = torch.empty(rows, dtype=torch.bfloat16, device=self.device)
        _arg(y, "y", torch.bfloat16, rows, self.device)
        check(_lib.lib().e4b_moe_fwd(ctypes.byref(self.desc), ctypes.byref(self._qgu),
                                     ctypes.byref(self._qdn), self._l(self._lgu), self._l(self._ldn),
                                     _ptr(x), _ptr(ids), _ptr(topw), _ptr(y), _ptr(self.ws),
                                     self.ws_bytes, _stream()), "e4b_moe_fwd")
        return y

    def forward_noalloc(self, x, ids, topw, y):
        """The forward through e4b_moe_fwd_noalloc: the library's per-GPU scratch array in place
        of this layer's workspace (inference layers only; y is caller-allocated)."""
        rows = (self.T, self.H)
        _arg(x, "x", torch.bfloat16, rows, self.device)
        self._routing(ids, topw)
        _arg(y, "y", torch.bfloat16, rows, self.device)
        check(_lib.lib().e4b_moe_fwd_noalloc(ctypes.byref(self.desc), ctypes.byref(self._qgu),
                                             ctypes.byref(self._qdn), self._l(self._lgu), self._l(self._ldn),
                                             _ptr(x), _ptr(ids), _ptr(topw), _ptr(y), _stream()),
              "e4b_moe_fwd_noalloc")
        return y

    def dgrad(self, ids, topw, dy, dx=None, d_topw=None, want_d_topw=True):
        rows = (self.T, self.H)
        _arg(dy, "dy", torch.bfloat16, rows, self.device)
        self._routing(ids, topw)
        if dx is None:
            dx = torch.empty(rows, dtype=torch.bfloat16, device=self.device)
        _arg(dx, "dx", torch.bfloat16, rows, self.device)
        if d_topw is None and want_d_topw:
            d_topw = torch.empty(self.T, self.topk, dtype=torch.float32, device=self.device)
        if d_topw is not None:
            _arg(d_topw, "d_topw", torch.float32, (self.T, self.topk), self.device)
        check(_lib.lib().e4b_moe_dgrad(ctypes.byref(self.desc), ctypes.byref(self._qgu),
                                       ctypes.byref(self._qdn), self._l(self._lgu), self._l(self._ldn),
                                       _ptr(ids), _ptr(topw), _ptr(dy), _ptr(dx), _ptr(d_topw),
                                       _ptr(self.ws), self.ws_bytes, _stream()), "e4b_moe_dgrad")
        return dx, d_topw

    def wgrad(self, x, out=None):
        dev = self.device
        E, H, I = self.E, self.H, self.I
        _arg(x, "x", torch.bfloat16, (self.T, H), dev)
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
        shapes = {}
        if self.l_gu is not None:
            shapes.update(dA_gu=(E, self.l_gu.r, H), dB_gu=(E, 2 * I, self.l_gu.r))
        if self.l_dn is not None:
            shapes.update(dA_dn=(E, self.l_dn.r, I), dB_dn=(E, H, self.l_dn.r))
        for k, shp in shapes.items():
            _arg(out.get(k), k, torch.float32, shp, dev)
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
