"""The C ABI without a GPU: the library loads, exports every symbol the header
declares, and rejects invalid arguments on the host before launching anything."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    from grouped_nf4_gemm_amd import _lib

    if not os.path.exists(_lib.SO_PATH):
        import __graft_entry__

        __graft_entry__.build()
    return _lib


def _header_symbols():
    text = open(os.path.join(ROOT, "include", "e4b.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(e4b_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    syms = _header_symbols()
    assert len(syms) >= 14
    lib = L.lib()
    for s in syms:
        assert hasattr(lib, s), s
    assert set(syms) == set(L.EXPORTS)


def test_version_and_status(L):
    assert L.version() >= 100
    assert L.status_str(0) == "ok"
    assert "workspace" in L.status_str(3)


def _desc(L, E=8, H=128, I=256, T=16, k=2, flags=1):
    return L.Desc(E, H, I, T, k, flags)


def _ws(L, d, l1=None, l2=None):
    n = ctypes.c_size_t()
    st = L.lib().e4b_moe_workspace_size(ctypes.byref(d), l1, l2, ctypes.byref(n))
    return st, n.value


def test_workspace_size_valid(L):
    d = _desc(L)
    lo = L.Lora(1, 2, 16, 2.0)
    st, n = _ws(L, d, ctypes.byref(lo), ctypes.byref(lo))
    assert st == 0 and n > 0
    st2, n2 = _ws(L, _desc(L, flags=0), ctypes.byref(lo), ctypes.byref(lo))
    assert st2 == 0 and n2 < n  # inference keeps no backward activations
    st3, n3 = _ws(L, _desc(L, T=0))
    assert st3 == 0


def test_expanded_stacks_workspace(L):
    """Large calls (more than 256 routed rows) reserve bf16 copies of both stacks (E*2I*H +
    E*H*I bf16 values) only when the caller asks for them with E4B_EXPAND; by default the
    stacks are decoded inside the GEMM tiles and no copy exists.  Calls of at most 256 rows
    never expand."""
    E, H, I = 4, 128, 256
    copies = 2 * (E * 2 * I * H + E * H * I)
    TRAIN, EXPAND = 1, 2
    _, big_default = _ws(L, _desc(L, E=E, H=H, I=I, T=2048, k=2, flags=TRAIN))
    _, big_forced = _ws(L, _desc(L, E=E, H=H, I=I, T=2048, k=2, flags=TRAIN | EXPAND))
    assert big_forced - big_default >= copies
    _, small_default = _ws(L, _desc(L, E=E, H=H, I=I, T=128, k=2, flags=TRAIN))     # 256 rows
    _, small_forced = _ws(L, _desc(L, E=E, H=H, I=I, T=128, k=2, flags=TRAIN | EXPAND))
    assert small_forced == small_default
    st, _ = _ws(L, _desc(L, E=E, H=H, I=I, T=2048, k=2, flags=TRAIN | 8))  # unknown flag bit
    assert st == L.E4B_ERR_INVALID_ARG


def test_separate_flag_accepted(L):
    """E4B_SEPARATE (the decode-shaped forward as six launches) is a known flag; it does not
    change the workspace size."""
    SEPARATE = 4
    _, n0 = _ws(L, _desc(L, T=16, k=2, flags=0))
    st, n1 = _ws(L, _desc(L, T=16, k=2, flags=SEPARATE))
    assert st == 0 and n1 == n0


@pytest.mark.parametrize("kw", [dict(H=100), dict(I=96), dict(E=0), dict(k=9), dict(k=0),
                                dict(T=-1), dict(E=2000, k=1), dict(flags=8)])
def test_bad_desc_rejected(L, kw):
    st, _ = _ws(L, _desc(L, **kw))
    assert st == L.E4B_ERR_INVALID_ARG


@pytest.mark.parametrize("r", [4, 12, 136, 0])
def test_bad_rank_rejected(L, r):
    lo = L.Lora(1, 2, r, 2.0)
    st, _ = _ws(L, _desc(L), ctypes.byref(lo), None)
    assert st == L.E4B_ERR_INVALID_ARG


def test_B_without_A_rejected(L):
    lo = L.Lora(None, 2, 16, 2.0)
    st, _ = _ws(L, _desc(L), ctypes.byref(lo), None)
    assert st == L.E4B_ERR_INVALID_ARG


def _qw(L, fmt, E, N, K, scale2=True):
    return L.QWeight(fmt, E, N, K, 0x1000, 0x2000, 0x3000 if scale2 else None)


def _fwd(L, d, qg, qd, ws_bytes, x=0x10, ids=0x20, topw=0x30, y=0x40, ws=0x50):
    return L.lib().e4b_moe_fwd(ctypes.byref(d), ctypes.byref(qg), ctypes.byref(qd), None, None, x, ids,
                               topw, y, ws, ws_bytes, None)


def test_fwd_rejections_launch_nothing(L):
    L.reset_stats()
    d = _desc(L)
    ok_gu, ok_dn = _qw(L, 0, 8, 512, 128), _qw(L, 0, 8, 128, 256)
    _, need = _ws(L, d)
    assert _fwd(L, d, ok_gu, ok_dn, need - 1) == L.E4B_ERR_WORKSPACE
    assert _fwd(L, d, ok_gu, ok_dn, need, ws=None) == L.E4B_ERR_WORKSPACE
    assert _fwd(L, d, ok_gu, ok_dn, need, x=None) == L.E4B_ERR_INVALID_ARG
    assert _fwd(L, d, ok_gu, ok_dn, need, ids=None) == L.E4B_ERR_INVALID_ARG
    assert _fwd(L, d, _qw(L, 0, 8, 256, 128), ok_dn, need) == L.E4B_ERR_INVALID_ARG  # wrong 2I
    assert _fwd(L, d, _qw(L, 0, 7, 512, 128), ok_dn, need) == L.E4B_ERR_INVALID_ARG  # wrong E
    assert _fwd(L, d, _qw(L, 5, 8, 512, 128), _qw(L, 5, 8, 128, 256), need) == L.E4B_ERR_UNSUPPORTED
    assert _fwd(L, d, _qw(L, 0, 8, 512, 128), _qw(L, 2, 8, 128, 256), need) == L.E4B_ERR_UNSUPPORTED
    assert _fwd(L, d, _qw(L, 1, 8, 512, 128, False), _qw(L, 1, 8, 128, 256, False), need) == \
        L.E4B_ERR_INVALID_ARG  # NF4_DQ needs scale2
    st = L.get_stats()
    assert st["launches_total"] == 0


def test_dgrad_needs_training_forward(L):
    L.reset_stats()
    d = _desc(L, flags=0)
    qg, qd = _qw(L, 0, 8, 512, 128), _qw(L, 0, 8, 128, 256)
    _, need = _ws(L, d)
    st = L.lib().e4b_moe_dgrad(ctypes.byref(d), ctypes.byref(qg), ctypes.byref(qd), None, None, 0x1, 0x2,
                               0x3, 0x4, None, 0x5, need, None)
    assert st == L.E4B_ERR_INVALID_ARG
    assert L.get_stats()["launches_total"] == 0


def test_quantize_and_dequant_rejections(L):
    lib = L.lib()
    assert lib.e4b_quantize(7, 1, 8, 64, 0x1, 0x2, 0x3, None, None) == L.E4B_ERR_UNSUPPORTED
    assert lib.e4b_quantize(5, 1, 8, 64, 0x1, 0x2, 0x3, None, None) == L.E4B_ERR_UNSUPPORTED
    assert lib.e4b_quantize(0, 1, 8, 96, 0x1, 0x2, 0x3, None, None) == L.E4B_ERR_INVALID_ARG
    assert lib.e4b_quantize(1, 1, 8, 64, 0x1, 0x2, 0x3, None, None) == L.E4B_ERR_INVALID_ARG
    q = L.QWeight(0, 2, 8, 64, 0x1, 0x2, None)
    assert lib.e4b_dequant(ctypes.byref(q), 2, 0x10, None, None) == L.E4B_ERR_INVALID_ARG
    assert lib.e4b_dequant(ctypes.byref(q), 0, None, None, None) == L.E4B_ERR_INVALID_ARG
    assert L.get_stats()["launches_total"] == 0


def test_router_rejections(L):
    """Router entry points check their sizes before any launch; T = 0 launches nothing."""
    lib = L.lib()
    bad = L.E4B_ERR_INVALID_ARG
    assert lib.e4b_router_topk(0x1, 4, 8, 9, 0x2, 0x3, None) == bad      # topk > E
    assert lib.e4b_router_topk(0x1, 4, 1025, 2, 0x2, 0x3, None) == bad   # E above the limit
    assert lib.e4b_router_topk(0x1, 4, 128, 65, 0x2, 0x3, None) == bad   # topk above the limit
    assert lib.e4b_router_topk(0x1, 4, 8, 0, 0x2, 0x3, None) == bad
    assert lib.e4b_router_topk(None, 4, 8, 2, 0x2, 0x3, None) == bad
    assert lib.e4b_router_topk(None, 0, 8, 2, None, None, None) == L.E4B_OK
    assert lib.e4b_router_bwd(0x1, 0x2, 0x3, -1, 8, 2, 0x4, None) == bad
    assert lib.e4b_router_bwd(0x1, None, 0x3, 4, 8, 2, 0x4, None) == bad
    assert lib.e4b_router_bwd(None, None, None, 0, 8, 2, None, None) == L.E4B_OK


def test_no_cpu_fallback_in_product():
    """The product package never imports the oracle."""
    pkg = os.path.join(ROOT, "grouped_nf4_gemm_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "oracle.h" not in text and "liboracle" not in text, f


def test_layer_argument_checks_cpu():
    """The Python layer checks dtype, shape and device of every tensor before its pointer
    reaches the library (a wrong dtype or a short tensor would make a kernel read or write
    past the allocation)."""
    import torch

    from grouped_nf4_gemm_amd.layer import _arg

    dev = torch.device("cpu")
    ok = torch.zeros(4, 2, dtype=torch.int32)
    assert _arg(ok, "ids", torch.int32, (4, 2), dev) is ok
    with pytest.raises(ValueError, match="int32"):
        _arg(ok.to(torch.int64), "ids", torch.int32, (4, 2), dev)  # torch.topk's default dtype
    with pytest.raises(ValueError, match="shape"):
        _arg(ok[:3], "ids", torch.int32, (4, 2), dev)
    with pytest.raises(ValueError, match="contiguous"):
        _arg(torch.zeros(2, 4, dtype=torch.int32).t(), "ids", torch.int32, (4, 2), dev)
    with pytest.raises(ValueError, match="tensor"):
        _arg(None, "x", torch.bfloat16, (4, 2), dev)


def test_code_table_rejections(L):
    """A code table that the format has no use for is refused before any launch: an absmax
    table on a plain NF4 or MXFP4 stack, a 4-bit codebook on an MXFP4 stack."""
    lib = L.lib()
    L.reset_stats()
    cases = [L.QWeight(0, 1, 8, 64, 0x1, 0x2, None, 0x3, None),        # NF4 + dq_table
             L.QWeight(2, 1, 8, 64, 0x1, 0x2, None, 0x3, None),        # MXFP4 + dq_table
             L.QWeight(2, 1, 8, 64, 0x1, 0x2, None, None, 0x4),        # MXFP4 + codebook
             L.QWeight(3, 1, 8, 64, 0x1, 0x2, None, None, 0x4),        # INT8 + codebook
             L.QWeight(4, 1, 8, 64, 0x1, 0x2, None, 0x3, None)]        # FP8 + dq_table
    for q in cases:
        assert lib.e4b_dequant(ctypes.byref(q), 0, 0x10, None, None) == L.E4B_ERR_INVALID_ARG
    ok = L.QWeight(1, 1, 8, 64, 0x1, 0x2, 0x5, 0x3, 0x4)               # NF4_DQ + both tables
    d = L.Desc(1, 64, 64, 0, 1, 0)
    n = ctypes.c_size_t()
    assert lib.e4b_moe_workspace_size(ctypes.byref(d), None, None, ctypes.byref(n)) == 0
    assert L.get_stats()["launches_total"] == 0
    del ok


def test_activation_checks(L):
    """The activation block is checked before any launch: the stock epilogue takes no biases,
    the clamped GLU needs a finite alpha and a finite positive limit, and an unknown kind is
    refused as unsupported."""
    lib = L.lib()

    def ws_status(act):
        d = L.Desc(4, 64, 64, 8, 2, 1, ctypes.pointer(act))
        n = ctypes.c_size_t()
        return lib.e4b_moe_workspace_size(ctypes.byref(d), None, None, ctypes.byref(n))

    assert ws_status(L.Act(1, 1.702, 7.0, 0x10, 0x20)) == L.E4B_OK
    assert ws_status(L.Act(1, 1.702, 7.0, None, None)) == L.E4B_OK
    assert ws_status(L.Act(0, 0.0, 0.0, None, None)) == L.E4B_OK
    assert ws_status(L.Act(0, 0.0, 0.0, 0x10, None)) == L.E4B_ERR_INVALID_ARG
    assert ws_status(L.Act(1, 1.702, 0.0, None, None)) == L.E4B_ERR_INVALID_ARG
    assert ws_status(L.Act(1, float("nan"), 7.0, None, None)) == L.E4B_ERR_INVALID_ARG
    assert ws_status(L.Act(1, 1.702, float("inf"), None, None)) == L.E4B_ERR_INVALID_ARG
    assert ws_status(L.Act(7, 1.0, 1.0, None, None)) == L.E4B_ERR_UNSUPPORTED
