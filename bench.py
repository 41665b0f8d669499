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
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="large")
    p.add_argument("--no-cpu-baseline", action="store_true")
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


def kernel_work(s, fam: str, M: int, touched: int) -> tuple[float, float]:
    """Algorithmic (flops, bytes) of ONE launch of a kernel family on workload s.
    flops = 2*rows*cols*reduction over the base and LoRA products the step performs
    on routed rows only; bytes = packed weights + scales of the `touched` experts (those
    with at least one routed row) read once + their adapter rows + the operand and output
    rows the kernel must touch."""
    E, H, I, r = touched, s.H, s.I, s.r
    wbytes_per_elem = 0.5 + (4.0 / 64 if s.fmt == "nf4" else 1.0 / 64 if s.fmt == "nf4_dq" else 1.0 / 32)
    if fam == "gemm_gate_up":
        fl = 2.0 * M * 2 * I * H + 2.0 * M * 2 * I * r
        by = E * 2 * I * H * wbytes_per_elem + E * 2 * I * r * 2 + M * H * 2 + M * I * 2 + M * r * 2
        if s.name != "large" and not s.name.startswith("decode"):
            by += M * 2 * I * 2  # saved pre-activations (training)
    elif fam == "gemm_gate_up_dgrad":
        fl = 2.0 * M * H * 2 * I + 2.0 * M * H * r
        by = E * 2 * I * H * wbytes_per_elem + M * 2 * I * 2 + M * H * 4
    elif fam == "gemm_down":
        fl = 2.0 * M * H * I + 2.0 * M * H * r
        by = E * H * I * wbytes_per_elem + E * H * r * 2 + M * I * 2 + M * r * 2 + M * H * 4
    elif fam == "gemm_down_dgrad":
        fl = 2.0 * M * I * H + 2.0 * M * I * r
        by = E * H * I * wbytes_per_elem + M * H * 2 + 2 * M * 2 * I * 2
    else:
        fl, by = 0.0, 0.0
    return fl, by


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
    import numpy as np
    import torch

    import synth
    from grouped_nf4_gemm_amd import LoRA, MoELayer, QStack, timing_enable, timing_read

    s = synth.WORKLOADS[a.workload]
    with_bwd = not s.name.startswith("decode")
    dev = "cuda"
    if a.copy_calib:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    inp = synth.make_inputs(s)
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
    layers = [MoELayer(w_gu, w_dn, l_gu, l_dn, s.T, s.k, train=with_bwd, expand=a.expand)]
    for _ in range(ncopy - 1):
        cq = lambda q: QStack(q.fmt, q.E, q.N, q.K, q.codes.clone(), q.scale.clone(),
                              None if q.scale2 is None else q.scale2.clone())
        cl = lambda l: LoRA(l.A.clone(), l.B.clone(), l.scaling)
        layers.append(MoELayer(cq(w_gu), cq(w_dn), cl(l_gu), cl(l_dn), s.T, s.k, train=False))
    layer = layers[0]
    y = torch.empty(s.T, s.H, dtype=torch.bfloat16, device=dev)
    dx = torch.empty_like(y)
    d_topw = torch.empty(s.T, s.k, dtype=torch.float32, device=dev)
    grads = None
    nstep = 0

    def step():
        nonlocal grads, nstep
        layer = layers[nstep % len(layers)]
        nstep += 1
        layer.forward(x, ids, topw, y)
        if with_bwd:
            layer.dgrad(ids, topw, dy, dx, d_topw)
            grads = layer.wgrad(x, grads)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    timing_read()  # drop warmup events
    timing_enable(True)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(a.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    timing_enable(False)
    per_kernel = timing_read()
    ms = ev0.elapsed_time(ev1) / a.steps
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
        reps = max(1, -(-a.steps // len(layers)))
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
    routed = s.M
    value = routed / (ms / 1e3)

    # dominant kernel and its roofline
    dom = max(per_kernel.items(), key=lambda kv: kv[1][1])
    dom_name, (dom_n, dom_ms) = dom
    avg_ms = dom_ms / dom_n
    touched = int(np.unique(inp.ids[(inp.ids >= 0) & (inp.ids < s.E)]).size)
    fl, by = kernel_work(s, dom_name, routed, touched)
    if s.name.startswith("decode"):
        roof = {"bound": "hbm", "achieved": by / (avg_ms / 1e3) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": fl / (avg_ms / 1e3) / 1e12, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["kernel"] = dom_name
    roof["avg_launch_ms"] = avg_ms
    roof["traffic"] = read_traffic(dom_name, s.name)

    out = {
        "metric": "routed tokens/s (NF4+LoRA grouped MoE layer, fwd+dgrad+wgrad step)" if with_bwd
        else "routed tokens/s (NF4+LoRA grouped MoE layer, forward)",
        "value": value, "unit": "routed tokens/s", "n_gpus": 1, "steps": graph_steps if use_graph else a.steps, "warmup": a.warmup,
        "ms_per_step": ms, "ms_per_step_eager": ms_eager,
        "timed": ("%d replays of a HIP graph of %d forwards" % (graph_steps // len(layers), len(layers)))
        if use_graph else "%d eager steps" % a.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded; random-init weights quantised to " + s.fmt + ")",
        "config": {"workload": s.name, "E": s.E, "H": s.H, "I": s.I, "T": s.T, "topk": s.k, "r": s.r,
                   "alpha": s.alpha, "weights": s.fmt, "global_batch": s.T, "parallelism": "none (1 GPU)",
                   "layer_copies": len(layers), "experts_touched": touched},
        "step_tflops": step_flops(s, with_bwd) / (ms / 1e3) / 1e12,
        "step_mfma_frac": step_flops(s, with_bwd) / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
        "wall_s": wall,
        "roofline": roof,
        "kernels_ms_per_step": {k: v[1] / a.steps for k, v in sorted(per_kernel.items(), key=lambda kv: -kv[1][1])},
    }
    out["router"] = router_timing(s)
    del layer, layers, w_gu, w_dn
    torch.cuda.empty_cache()
    if not a.no_cpu_baseline:
        n_tok = a.cpu_sample_tokens or (320 if with_bwd else 16)
        out["cpu_baseline"] = cpu_baseline(s, inp, n_tok)
        out["gpu_over_cpu"] = out["value"] / out["cpu_baseline"]["value"]
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
