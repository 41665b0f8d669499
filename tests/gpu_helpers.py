"""Helpers shared by the GPU parity tests: upload the seeded inputs, run the
library through its C ABI, and compare against the oracle."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth
from grouped_nf4_gemm_amd import LoRA, MoELayer, QStack

MAX_REL = 2e-2   # max|gpu - ref| <= MAX_REL * max|ref|
L1_REL = 5e-3    # sum|gpu - ref| <= L1_REL * sum|ref|


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need an MI355X; run them with -m gpu on a GPU box")


def bf16_to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def close_stats(gpu: np.ndarray, ref: np.ndarray):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(gpu - ref)
    mx = np.abs(ref).max() if ref.size else 0.0
    l1 = np.abs(ref).sum()
    return (err.max() / mx if mx > 0 else float(err.max() if err.size else 0.0),
            err.sum() / l1 if l1 > 0 else float(err.sum()))


def assert_close(gpu, ref, name: str):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (name, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{name}: non-finite GPU values"
    if ref.size == 0:
        return
    if np.abs(ref).max() == 0:
        assert np.abs(gpu).max() == 0, f"{name}: reference is exactly zero, GPU is not"
        return
    mrel, l1 = close_stats(gpu, ref)
    assert mrel <= MAX_REL and l1 <= L1_REL, f"{name}: max-rel {mrel:.3e}, rel-L1 {l1:.3e}"


class Case:
    """One layer call: host inputs, oracle-quantised stacks, and device copies."""

    def __init__(self, inp: synth.LayerInputs, lora: bool = True, train: bool = True, expand=None,
                 dq_table=None, codebook=None):
        """dq_table / codebook (fp32 numpy arrays): the stacks' own code tables, read by
        both sides in place of the built-in ones (the bytes are quantised against the
        built-in tables either way)."""
        s = inp.shape
        self.inp, self.s = inp, s
        self.q1 = oracle.quantize(s.fmt, inp.W1).with_tables(dq_table, codebook)
        self.q2 = oracle.quantize(s.fmt, inp.W2).with_tables(dq_table, codebook)
        dev = "cuda"
        self.w_gu = QStack.from_host(s.fmt, s.E, 2 * s.I, s.H, self.q1.codes, self.q1.scale, self.q1.scale2,
                                     dq_table=dq_table, codebook=codebook)
        self.w_dn = QStack.from_host(s.fmt, s.E, s.H, s.I, self.q2.codes, self.q2.scale, self.q2.scale2,
                                     dq_table=dq_table, codebook=codebook)
        b16 = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        self.l_gu = LoRA(b16(inp.A1), b16(inp.B1), s.scaling) if lora else None
        self.l_dn = LoRA(b16(inp.A2), b16(inp.B2), s.scaling) if lora else None
        self.x = b16(inp.x)
        self.dy = b16(inp.dy)
        self.ids = torch.from_numpy(inp.ids).to(dev)
        self.topw = torch.from_numpy(inp.topw).to(dev)
        self.layer = MoELayer(self.w_gu, self.w_dn, self.l_gu, self.l_dn, s.T, s.k, train=train,
                              expand=expand)
        self.lora = lora

    def oracle_layer(self):
        return oracle.layer_from_inputs(self.inp, self.q1, self.q2, lora=self.lora)

    def run(self, dgrad=True, wgrad=True, dy=None):
        y = self.layer.forward(self.x, self.ids, self.topw)
        out = {"y": y}
        if dgrad:
            dx, dw = self.layer.dgrad(self.ids, self.topw, self.dy if dy is None else dy)
            out["dx"], out["dw"] = dx, dw
            if wgrad and self.lora:
                out.update(self.layer.wgrad(self.x))
        torch.cuda.synchronize()
        return out
