"""ctypes binding over libe4b.so (argument marshalling only).

Every computation runs in the HIP library.  If libe4b.so is missing this module
raises on import of the binding: there is no slower path to fall back to.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
SO_PATH = os.path.join(_PKG, "libe4b.so")

E4B_OK, E4B_ERR_INVALID_ARG, E4B_ERR_UNSUPPORTED, E4B_ERR_WORKSPACE, E4B_ERR_HIP = range(5)
FMT = {"nf4": 0, "nf4_dq": 1, "mxfp4": 2, "int8": 3, "fp8": 4}
E4B_TRAIN = 1
E4B_EXPAND = 2
E4B_SEPARATE = 4

EXPORTS = [
    "e4b_version", "e4b_status_str", "e4b_moe_workspace_size", "e4b_moe_fwd", "e4b_moe_dgrad",
    "e4b_lora_wgrad", "e4b_moe_route", "e4b_dequant", "e4b_quantize", "e4b_moe_check",
    "e4b_get_stats", "e4b_reset_stats", "e4b_timing_enable", "e4b_timing_read",
    "e4b_router_topk", "e4b_router_bwd", "e4b_moe_fwd_noalloc",
]
NOALLOC_SCRATCH_BYTES = 64 << 20


class E4BError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} (status {status})")


class QWeight(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("E", ctypes.c_int32), ("N", ctypes.c_int32),
                ("K", ctypes.c_int32), ("codes", ctypes.c_void_p), ("scale", ctypes.c_void_p),
                ("scale2", ctypes.c_void_p), ("dq_table", ctypes.c_void_p), ("codebook", ctypes.c_void_p)]


class Lora(ctypes.Structure):
    _fields_ = [("A", ctypes.c_void_p), ("B", ctypes.c_void_p), ("r", ctypes.c_int32),
                ("scaling", ctypes.c_float)]


ACT = {"swiglu": 0, "clamped_glu": 1}


class Act(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("alpha", ctypes.c_float), ("limit", ctypes.c_float),
                ("b_gu", ctypes.c_void_p), ("b_dn", ctypes.c_void_p)]


class Desc(ctypes.Structure):
    _fields_ = [("E", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("T", ctypes.c_int32), ("topk", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("act", ctypes.POINTER(Act))]


class Stats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "launches_total", "route", "lora_a", "gemm_gate_up", "gemm_down", "combine",
        "combine_bwd", "gemm_down_dgrad", "gemm_gate_up_dgrad", "unpermute", "wgrad", "quant",
        "dequant", "expand", "router", "fallbacks")]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(SO_PATH):
            raise RuntimeError(f"libe4b.so not built at {SO_PATH}; run __graft_entry__.build()")
        L = ctypes.CDLL(SO_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        P = ctypes.POINTER
        L.e4b_version.restype = i32
        L.e4b_status_str.restype = ctypes.c_char_p
        L.e4b_status_str.argtypes = [i32]
        L.e4b_moe_workspace_size.restype = i32
        L.e4b_moe_workspace_size.argtypes = [P(Desc), P(Lora), P(Lora), P(sz)]
        L.e4b_moe_fwd.restype = i32
        L.e4b_moe_fwd.argtypes = [P(Desc), P(QWeight), P(QWeight), P(Lora), P(Lora), vp, vp, vp, vp,
                                  vp, sz, vp]
        L.e4b_moe_fwd_noalloc.restype = i32
        L.e4b_moe_fwd_noalloc.argtypes = [P(Desc), P(QWeight), P(QWeight), P(Lora), P(Lora), vp, vp, vp, vp, vp]
        L.e4b_moe_dgrad.restype = i32
        L.e4b_moe_dgrad.argtypes = [P(Desc), P(QWeight), P(QWeight), P(Lora), P(Lora), vp, vp, vp, vp,
                                    vp, vp, sz, vp]
        L.e4b_lora_wgrad.restype = i32
        L.e4b_lora_wgrad.argtypes = [P(Desc), P(Lora), P(Lora), vp, vp, sz, vp, vp, vp, vp, vp]
        L.e4b_moe_route.restype = i32
        L.e4b_moe_route.argtypes = [P(Desc), vp, vp, vp, vp, vp, vp]
        L.e4b_router_topk.restype = i32
        L.e4b_router_topk.argtypes = [vp, i32, i32, i32, vp, vp, vp]
        L.e4b_router_bwd.restype = i32
        L.e4b_router_bwd.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp]
        L.e4b_dequant.restype = i32
        L.e4b_dequant.argtypes = [P(QWeight), i32, vp, vp, vp]
        L.e4b_quantize.restype = i32
        L.e4b_quantize.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp]
        L.e4b_moe_check.restype = i32
        L.e4b_moe_check.argtypes = [P(Desc), vp, vp, P(i32)]
        L.e4b_get_stats.restype = i32
        L.e4b_get_stats.argtypes = [P(Stats)]
        L.e4b_reset_stats.restype = None
        L.e4b_timing_enable.restype = i32
        L.e4b_timing_enable.argtypes = [i32]
        L.e4b_timing_read.restype = i32
        L.e4b_timing_read.argtypes = [i32, vp, P(ctypes.c_int64), P(ctypes.c_double), P(i32)]
        _lib = L
    return _lib


def status_str(s: int) -> str:
    return lib().e4b_status_str(int(s)).decode()


def check(status: int, where: str) -> None:
    if status != E4B_OK:
        raise E4BError(status, where)


def version() -> int:
    return lib().e4b_version()


def get_stats() -> dict:
    s = Stats()
    check(lib().e4b_get_stats(ctypes.byref(s)), "e4b_get_stats")
    return {n: getattr(s, n) for n, _ in Stats._fields_}


def reset_stats() -> None:
    lib().e4b_reset_stats()


def timing_enable(on: bool) -> None:
    check(lib().e4b_timing_enable(1 if on else 0), "e4b_timing_enable")


def timing_read() -> dict:
    """Per kernel family: (launches, total ms) since the last read.  Synchronises."""
    n_max = 32
    names = (ctypes.c_char * 32 * n_max)()
    launches = (ctypes.c_int64 * n_max)()
    ms = (ctypes.c_double * n_max)()
    n = ctypes.c_int32()
    check(lib().e4b_timing_read(n_max, ctypes.cast(names, ctypes.c_void_p), launches, ms,
                                ctypes.byref(n)), "e4b_timing_read")
    return {names[i].value.decode(): (launches[i], ms[i]) for i in range(min(n.value, n_max))}
