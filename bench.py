"""Throughput of the routed-expert MoE layer (NF4 + per-expert LoRA) on one MI355X.

One step = forward + input gradient + LoRA weight gradients of the layer over one
batch of seeded synthetic input, inputs resident in HBM.  Prints ONE JSON line.

Default workload ("large"): E=8, H=4096, I=14336, top-2, T=16384 tokens, LoRA
r=64 / alpha=128 on gate_up and down, NF4 blocks of 64 with double-quantised
absmax, router logits N(0,1) + per-expert bias N(0,0.5).  Other workloads of
synth.WORKLOADS can be timed with --workload (decode-t* run the forward only).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="large")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-secondary", action="store_true",
                   help="large workload: skip the decode, many-small and mxfp4 lines")
    p.add_argument("--cpu-sample-tokens", type=int, default=0, help="0 = automatic")
    p.add_argument("--copy-calib", action="store_true",
                   help="run a plain 256 MiB device copy first (HBM counter calibration)")
    p.add_argument("--summarize-stats", nargs=2, metavar=("STATS_CSV", "OUT_TXT"),
                   help="write a text summary of a rocprofv3 --stats kernel_stats.csv and exit")
    p.add_argument("--summarize-pmc", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "OUT_TXT"),
                   help="write per-kernel HBM traffic from two rocprofv3 --pmc runs and exit")
    p.add_argument("--command", default="", help="command line recorded in a summary")
    p.add_argument("--expand", action="store_true",
                   help="large calls: the forward streams bf16 copies of the stacks instead of decoding them in the tile")
    p.add_argument("--separate", action="store_true",
                   help="decode-shaped forward as six launches instead of two")
    p.add_argument("--graph", choices=("auto", "on", "off"), default="auto",
                   help="time forward-only steps as replays of one captured HIP graph "
                        "(auto: on for the decode-shaped workloads)")
    return p.parse_args()


def csrc_sha() -> str:
    h = hashlib.sha256()
    d = os.path.join(ROOT, "grouped_nf4_gemm_amd", "csrc")
    for f in sorted(os.listdir(d)):
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


RIDGE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)  # flop/byte where the two roofs meet


def step_work(s, fam: str, touched: int, train: bool, nsplit: int = 1) -> tuple[float, float]:
    """Algorithmic (flops, bytes) of ONE STEP's launches of a kernel family on workload s.
    flops = 2*rows*cols*reduction over the base and LoRA products on routed rows only (no tile
    padding); bytes = every operand and output the family must touch once: packed weights and
    scales of the `touched` experts (those with routed rows), their adapter rows, activation
    rows in and out.  The same rules hold for every workload (training or forward only)."""
    M, T, k, E, H, I, r = s.M, s.T, s.k, touched, s.H, s.I, s.r
    wb = 0.5 + (4.0 / 64 if s.fmt == "nf4" else 1.0 / 64 if s.fmt == "nf4_dq" else 1.0 / 32)
    if s.fmt in ("int8", "fp8"):
        wb = 1.0 + 4.0 / 64
    bf, f4 = 2, 4
    if fam == "gemm_gate_up":
        fl = 2.0 * M * 2 * I * H + 2.0 * M * 2 * I * r
        by = E * 2 * I * H * wb + E * 2 * I * r * bf + M * H * bf + M * r * bf + M * I * bf
        by += M * 2 * I * bf if train else 0  # saved pre-activation
    elif fam == "gemm_down":
        fl = 2.0 * M * H * I + 2.0 * M * H * r
        by = E * H * I * wb + E * H * r * bf + M * I * bf + M * r * bf + M * H * f4 * nsplit
    elif fam == "gemm_down_dgrad":
        fl = 2.0 * M * I * H + 2.0 * M * I * r
        by = E * H * I * wb + E * I * r * bf + M * H * bf + M * r * bf + 2 * M * 2 * I * bf
    elif fam == "gemm_gate_up_dgrad":
        fl = 2.0 * M * H * 2 * I + 2.0 * M * H * r
        by = E * 2 * I * H * wb + E * H * r * bf + M * 2 * I * bf + M * r * bf + M * H * f4
    elif fam == "lora_a":  # z1 = A1 x, z2 = A2 h (+ u2 = B2^T dO, u1 = B1^T dG when training)
        fl = 2.0 * M * r * (H + I) + (2.0 * M * r * (H + 2 * I) if train else 0)
        by = M * (H + I) * bf + E * r * (H + I) * bf + 2 * M * r * bf
        if train:
            by += M * (H + 2 * I) * bf + E * r * (H + 2 * I) * bf + 2 * M * r * bf
    elif fam == "wgrad":  # dB1, dA1, dB2, dA2: reductions over each expert's rows
        fl = 2.0 * M * r * (2 * I + H + H + I)
        by = M * (2 * I + H + H + I) * bf + 4 * M * r * bf + s.E * r * (2 * I + H + H + I) * f4
    elif fam == "combine":
        fl, by = 0.0, M * H * f4 * nsplit + T * H * bf + T * k * 8
    elif fam == "combine_bwd":
        fl, by = 0.0, T * H * bf + M * H * f4 + M * H * bf + T * k * 12
    elif fam == "unpermute":
        fl, by = 0.0, M * H * f4 + T * H * bf + T * k * 4
    elif fam == "route":
        fl, by = 0.0, M * 4 + 2 * M * 4 + 2 * (s.E + 1) * 4
    elif fam == "transpose":  # the four adapter matrices read and written once
        fl, by = 0.0, 2 * s.E * r * (2 * I + H + H + I) * bf
    elif fam == "expand":  # packed stacks in, bf16 copies out
        fl, by = 0.0, s.E * 3 * I * H * (wb + bf)
    else:
        raise KeyError(f"no algorithmic work formula for kernel family {fam!r}")
    return fl, by


def roof_of(fl: float, by: float, ms: float) -> dict:
    """Roofline entry of `ms` milliseconds of work: bound by MFMA (bf16 peak) when the
    arithmetic intensity is above the ridge, else by HBM."""
    sec = ms / 1e3
    if fl > 0 and fl / max(by, 1.0) >= RIDGE:
        return {"bound": "mfma", "achieved": fl / sec / 1e12, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": fl / sec / 1e12 / PEAK_BF16_TFLOPS}
    return {"bound": "hbm", "achieved": by / sec / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": by / sec / 1e9 / PEAK_HBM_GBS}


def step_flops(s, with_bwd: bool) -> float:
    M, H, I, r = s.M, s.H, s.I, s.r
    fwd = 2.0 * M * (2 * I * H + H * I) + 2.0 * M * r * (H + 2 * I) + 2.0 * M * r * (I + H)
    if not with_bwd:
        return fwd
    dgrad = 2.0 * M * (H * I + 2 * I * H) + 2.0 * M * r * (H + I) + 2.0 * M * r * (2 * I + H)
    wgrad = 2.0 * M * r * (2 * I + H + H + I)
    return fwd + dgrad + wgrad


def cpu_baseline(s, inp, n_tokens: int):
    """The oracle, untuned, on a bounded token sample of the same workload."""
    import numpy as np

    import oracle

    oracle.build(force=False)
    rng = np.random.default_rng(0)
    toks = np.sort(rng.choice(s.T, size=min(n_tokens, s.T), replace=False))
    q1 = oracle.quantize(s.fmt, inp.W1)
    q2 = oracle.quantize(s.fmt, inp.W2)
    L = oracle.layer_from_inputs(inp, q1, q2)
    t0 = time.perf_counter()
    oracle.moe_fwd(L, tokens=toks)
    with_bwd = not s.name.startswith("decode")
    if with_bwd:
        oracle.moe_bwd(L, inp.dy, tokens=toks)
    dt = time.perf_counter() - t0
    rows = int((inp.ids[toks] >= 0).sum())
    cores = int(os.environ.get("OMP_NUM_THREADS", 0)) or len(os.sched_getaffinity(0))
    return {"value": rows / dt, "unit": "routed tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{len(toks)} of {s.T} tokens ({rows} routed rows), "
                      f"{'fwd+dgrad+wgrad' if with_bwd else 'fwd'}, {dt:.1f} s wall"}


COPY_BYTES = 256 << 20


def summarize_stats(csv_path: str, out_path: str, command: str) -> None:
    import csv

    rows = list(csv.DictReader(open(csv_path)))
    lines = [f"# rocprofv3 kernel statistics", f"# command: {command}", f"# source: {os.path.basename(csv_path)}",
             f"{'kernel':60s} {'calls':>6s} {'total_ms':>10s} {'avg_us':>10s} {'pct':>6s}"]
    for r in rows:
        name = r.get("Name", r.get("KernelName", "?"))
        short = name.split("(")[0][:60]
        lines.append(f"{short:60s} {int(r['Calls']):6d} {float(r['TotalDurationNs'])/1e6:10.3f} "
                     f"{float(r['AverageNs'])/1e3:10.1f} {float(r['Percentage']):6.2f}")
    open(out_path, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _pmc_per_kernel(csv_path: str) -> dict:
    import csv

    acc: dict = {}
    for r in csv.DictReader(open(csv_path)):
        name = r.get("Kernel_Name", r.get("KernelName", "?")).split("(")[0]
        v = float(r.get("Counter_Value", r.get("Value", 0)))
        key = (name, r.get("Dispatch_Id", r.get("Correlation_Id", "")))
        acc[key] = acc.get(key, 0.0) + v
    out: dict = {}
    for (name, _), v in acc.items():
        n, tot = out.get(name, (0, 0.0))
        out[name] = (n + 1, tot + v)
    return {k: (n, tot / n) for k, (n, tot) in out.items()}


def summarize_pmc(fetch_csv: str, write_csv: str, out_path: str, command: str) -> None:
    """FETCH_SIZE / WRITE_SIZE are KiB per dispatch; scale each by the ratio of the known
    bytes of a plain device copy to what the same counter reads for that copy."""
    f = _pmc_per_kernel(fetch_csv)
    w = _pmc_per_kernel(write_csv)
    copy = [k for k in f if "copy" in k.lower() or "elementwise" in k.lower()]
    ref = max(copy, key=lambda k: f[k][1]) if copy else None
    f_scale = COPY_BYTES / (f[ref][1] * 1024) if ref else 1.0
    w_scale = COPY_BYTES / (w[ref][1] * 1024) if ref and ref in w and w[ref][1] > 0 else 1.0
    lines = ["# HBM traffic per dispatch from rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE",
             f"# command: {command}",
             f"# calibration kernel: {ref} ({COPY_BYTES} bytes read and written); "
             f"fetch scale {f_scale:.4f}, write scale {w_scale:.4f}",
             f"csrc_sha: {csrc_sha()}",
             f"{'kernel':60s} {'dispatches':>10s} {'fetch_MB':>10s} {'write_MB':>10s}"]
    for k in sorted(f, key=lambda k: -f[k][1]):
        fb = f[k][1] * 1024 * f_scale
        wb = w.get(k, (0, 0.0))[1] * 1024 * w_scale
        lines.append(f"{k[:60]:60s} {f[k][0]:10d} {fb/1e6:10.2f} {wb/1e6:10.2f}")
    open(out_path, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


# kernel family (as the library's event timing names it) -> kernel symbol fragments: the
# kernel that decodes in the tile, and the one over bf16 copies of the stacks (--expand)
FAMILY_SYMBOL = {
    "gemm_gate_up": ("gemm_ws_kernel<0, 2,", "gemm_x_kernel<false, 2,"),
    "gemm_down": ("gemm_ws_kernel<0, 0,", "gemm_x_kernel<false, 0,"),
    "gemm_down_dgrad": ("gemm_ws_kernel<1, 3,", "gemm_x_kernel<true, 3,"),
    "gemm_gate_up_dgrad": ("gemm_ws_kernel<1, 0,", "gemm_x_kernel<true, 0,"),
}


def read_traffic(family: str, workload: str):
    """HBM bytes per launch (fetch + write) of a kernel family from the committed counter
    summary of this workload, if it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    sym = FAMILY_SYMBOL.get(family)
    if not os.path.exists(path) or sym is None:
        return None
    lines = open(path).read().splitlines()
    sha = next((l.split(":", 1)[1].strip() for l in lines if l.startswith("csrc_sha:")), None)
    if sha != csrc_sha():
        return None
    for frag in sym:
        for line in lines:
            parts = line.split()
            if frag in line and len(parts) >= 4:
                try:
                    return (float(parts[-2]) + float(parts[-1])) * 1e6
                except ValueError:
                    continue
    return None


def router_timing(s, reps: int = 50) -> dict:
    """The router step on this workload's T x E fp32 logits (outside the timed layer step):
    average of `reps` launches each of e4b_router_topk and e4b_router_bwd, HIP events on the
    launch stream; HBM bytes = logits (+ d logits) + ids and weights."""
    import torch
    from grouped_nf4_gemm_amd import router_bwd, router_topk
    if s.T == 0:
        return {}
    g = torch.Generator(device="cuda").manual_seed(5)
    logits = torch.randn(s.T, s.E, device="cuda", generator=g)
    ids, w = router_topk(logits, s.k)
    dw = torch.randn(s.T, s.k, device="cuda", generator=g)
    res = {}
    for name, fn, nbytes in (("fwd", lambda: router_topk(logits, s.k), s.T * s.E * 4 + s.T * s.k * 8),
                             ("bwd", lambda: router_bwd(w, dw, ids, s.E), s.T * s.k * 12 + s.T * s.E * 4)):
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        res[name + "_us"] = us
        res[name + "_hbm_frac"] = nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS
    return res


def measure(s, a, inp, steps: int, warmup: int, kernel_steps: int) -> dict:
    """Time `steps` steps of workload s (inputs resident in HBM) and return the result fields:
    ms/step from HIP events around the timed steps (graph replays for forward-only workloads),
    then, in a separate pass outside that window, per-kernel-family times from the library's
    own events on its launch stream, and the roofline of the dominant family."""
    import numpy as np
    import torch

    from grouped_nf4_gemm_amd import LoRA, MoELayer, QStack, timing_enable, timing_read

    with_bwd = not s.name.startswith("decode")
    dev = "cuda"
    b16 = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
    w_gu = QStack.quantize(s.fmt, torch.from_numpy(inp.W1).to(dev))
    w_dn = QStack.quantize(s.fmt, torch.from_numpy(inp.W2).to(dev))
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    l_gu = LoRA(b16(inp.A1), b16(inp.B1), s.scaling)
    l_dn = LoRA(b16(inp.A2), b16(inp.B2), s.scaling)
    x, dy = b16(inp.x), b16(inp.dy)
    ids, topw = torch.from_numpy(inp.ids).to(dev), torch.from_numpy(inp.topw).to(dev)
    # Forward-only (decode-shaped) steps rotate over separate resident copies of the layer
    # (> 2 GB in all), so the 256 MB last-level cache cannot serve the weights of a step
    # from the previous ones; every copy holds the same bytes.
    ncopy = 1 if with_bwd else max(1, -(-2_500_000_000 // (w_gu.codes.numel() + w_dn.codes.numel())))
    layers = [MoELayer(w_gu, w_dn, l_gu, l_dn, s.T, s.k, train=with_bwd, expand=a.expand, separate=a.separate)]
    for _ in range(ncopy - 1):
        cq = lambda q: QStack(q.fmt, q.E, q.N, q.K, q.codes.clone(), q.scale.clone(),
                              None if q.scale2 is None else q.scale2.clone())
        cl = lambda l: LoRA(l.A.clone(), l.B.clone(), l.scaling)
        layers.append(MoELayer(cq(w_gu), cq(w_dn), cl(l_gu), cl(l_dn), s.T, s.k, train=False, separate=a.separate))
    y = torch.empty(s.T, s.H, dtype=torch.bfloat16, device=dev)
    dx = torch.empty_like(y)
    d_topw = torch.empty(s.T, s.k, dtype=torch.float32, device=dev)
    state = {"grads": None, "n": 0}

    def step():
        layer = layers[state["n"] % len(layers)]
        state["n"] += 1
        layer.forward(x, ids, topw, y)
        if with_bwd:
            layer.dgrad(ids, topw, dy, dx, d_topw)
            state["grads"] = layer.wgrad(x, state["grads"])

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / steps
    ms_eager = ms
    use_graph = a.graph == "on" or (a.graph == "auto" and not with_bwd)
    graph_steps = 0
    if use_graph:
        # One capture holds a forward on every layer copy in rotation order; its replays are
        # the timed steps (launch gaps of the eager stream removed).  The replayed output
        # must equal the eager one: every copy holds the same bytes.
        if with_bwd:
            raise SystemExit("--graph applies to forward-only workloads")
        y_ref = y.clone()
        reps = max(1, -(-steps // len(layers)))
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for lyr in layers:
                lyr.forward(x, ids, topw, y)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for lyr in layers:
                lyr.forward(x, ids, topw, y)
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()
        if not torch.equal(y, y_ref):
            raise SystemExit("graph replay output differs from the eager forward")
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(reps):
            graph.replay()
        g1.record()
        torch.cuda.synchronize()
        graph_steps = reps * len(layers)
        ms = g0.elapsed_time(g1) / graph_steps
        del graph
    # per-kernel pass, outside the timed window
    timing_read()
    timing_enable(True)
    for _ in range(kernel_steps):
        step()
    torch.cuda.synchronize()
    timing_enable(False)
    per_kernel = timing_read()
    touched = int(np.unique(inp.ids[(inp.ids >= 0) & (inp.ids < s.E)]).size)
    kernels = {}
    for fam, (n, tot) in sorted(per_kernel.items(), key=lambda kv: -kv[1][1]):
        kms = tot / kernel_steps
        fl, by = step_work(s, fam, touched, with_bwd)
        r = roof_of(fl, by, kms)
        kernels[fam] = {"ms_per_step": kms, "launches_per_step": n / kernel_steps, "bound": r["bound"],
                        "frac": r["frac"]}
    dom = max(kernels, key=lambda f: kernels[f]["ms_per_step"])
    n_dom = kernels[dom]["launches_per_step"]
    avg_ms = kernels[dom]["ms_per_step"] / n_dom
    fl, by = step_work(s, dom, touched, with_bwd)
    roof = roof_of(fl / n_dom, by / n_dom, avg_ms)
    roof.update({"kernel": dom, "avg_launch_ms": avg_ms, "traffic": read_traffic(dom, s.name)})
    del layers, w_gu, w_dn
    torch.cuda.empty_cache()
    return {
        "value": s.M / (ms / 1e3), "ms_per_step": ms, "ms_per_step_eager": ms_eager,
        "steps": graph_steps if use_graph else steps,
        "timed": ("%d replays of a HIP graph of %d forwards" % (graph_steps // ncopy, ncopy))
        if use_graph else "%d eager steps" % steps,
        "touched": touched, "layer_copies": ncopy, "wall_s": wall,
        "step_tflops": step_flops(s, with_bwd) / (ms / 1e3) / 1e12,
        "roofline": roof, "kernels": kernels,
    }


SECONDARY = ("decode-t1", "decode-t8", "decode-t64", "many-small", "mxfp4")


def main():
    a = parse()
    if a.summarize_stats:
        summarize_stats(*a.summarize_stats, a.command)
        return
    if a.summarize_pmc:
        summarize_pmc(*a.summarize_pmc, a.command)
        return
    if a.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; multi-GPU sharding is described in "
                                   "DESIGN.md and not implemented", "n_gpus": a.gpus}))
        sys.exit(2)
    import torch

    import synth

    s = synth.WORKLOADS[a.workload]
    with_bwd = not s.name.startswith("decode")
    if a.copy_calib:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    inp = synth.make_inputs(s)
    res = measure(s, a, inp, a.steps, a.warmup, min(a.steps, 5))
    out = {
        "metric": "routed tokens/s (NF4+LoRA grouped MoE layer, fwd+dgrad+wgrad step)" if with_bwd
        else "routed tokens/s (NF4+LoRA grouped MoE layer, forward)",
        "value": res["value"], "unit": "routed tokens/s", "n_gpus": 1, "steps": res["steps"],
        "warmup": a.warmup, "ms_per_step": res["ms_per_step"], "ms_per_step_eager": res["ms_per_step_eager"],
        "timed": res["timed"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded; random-init weights quantised to " + s.fmt + ")",
        "config": {"workload": s.name, "E": s.E, "H": s.H, "I": s.I, "T": s.T, "topk": s.k, "r": s.r,
                   "alpha": s.alpha, "weights": s.fmt, "global_batch": s.T, "parallelism": "none (1 GPU)",
                   "layer_copies": res["layer_copies"], "experts_touched": res["touched"]},
        "step_tflops": res["step_tflops"], "step_mfma_frac": res["step_tflops"] / PEAK_BF16_TFLOPS,
        "wall_s": res["wall_s"], "roofline": res["roofline"],
        "kernels": {k: {kk: round(vv, 5) for kk, vv in v.items() if kk != "bound"} | {"bound": v["bound"]}
                    for k, v in res["kernels"].items()},
    }
    out["router"] = router_timing(s)
    if a.workload == "large" and not a.no_secondary:
        # the other configurations of the same layer, measured in the same run (their own
        # inputs; the three decode batch sizes share one set of weights)
        sec = {}
        dec_w = None
        for name in SECONDARY:
            s2 = synth.WORKLOADS[name]
            if name.startswith("decode"):
                inp2 = synth.make_inputs(s2, weights=dec_w is None)
                if dec_w is None:
                    dec_w = (inp2.W1, inp2.W2)
                inp2.W1, inp2.W2 = dec_w
                r2 = measure(s2, a, inp2, 40, 5, 5)
            else:
                r2 = measure(s2, a, synth.make_inputs(s2), 20, 3, 5)
            top = sorted(r2["kernels"].items(), key=lambda kv: -kv[1]["ms_per_step"])[:4]
            sec[name] = {"value": r2["value"], "ms_per_step": r2["ms_per_step"], "timed": r2["timed"],
                         "roofline": {k: r2["roofline"][k] for k in ("kernel", "bound", "frac", "achieved", "unit",
                                                                    "avg_launch_ms")},
                         "kernels": {k: {"ms_per_step": round(v["ms_per_step"], 5), "frac": round(v["frac"], 4)}
                                     for k, v in top}}
            print(f"# secondary {name}: {r2['ms_per_step']:.4f} ms/step, {r2['roofline']['kernel']} "
                  f"{r2['roofline']['frac']:.3f} of {r2['roofline']['bound']}", file=sys.stderr, flush=True)
        out["secondary"] = sec
    if not a.no_cpu_baseline:
        n_tok = a.cpu_sample_tokens or (320 if with_bwd else 16)
        out["cpu_baseline"] = cpu_baseline(s, inp, n_tok)
        out["gpu_over_cpu"] = out["value"] / out["cpu_baseline"]["value"]
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
