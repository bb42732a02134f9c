#!/usr/bin/env python3
"""Throughput of the streaming CG tensor-product convolution on one MI355X.

A step is one pass of the workload's hot path over its synthetic radius graph:
forward (receiver stream + contraction) and backward w.r.t. x, W and
positions; the "force" workload adds the double backward of the force loss.
Inputs are resident in HBM before the timed region.  Prints ONE JSON line with
edges/s (whole job), per-pass throughput, peak workspace bytes, the dominant
kernel's roofline (algorithmic FLOPs or bytes per launch over its HIP-event
duration) and the CPU oracle's throughput on a bounded sample.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload molecular]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "edges/sec fwd and fwd+bwd per config; % of HBM/MFMA roofline; peak bytes"
PEAK = {"hbm": (8000.0, "GB/s"), "mfma": (157.3, "TFLOP/s"), "alu": (157.3, "TFLOP/s")}


def plan_counts(plan):
    """Per-path (l1, l2, l3, nnz) from the plan's own tables."""
    import numpy as np

    out = []
    for i in range(plan.num_paths):
        (l1, l2, l3), _ = plan.path(i)
        out.append((l1, l2, l3, int((np.abs(plan.cg(i)) > 1e-12).sum())))
    return out


def algorithmic(plan, paths, N, E, xbytes):
    """Algorithmic FLOPs and compulsory HBM bytes per launch of each kernel class."""
    K, Ci, Co = plan.num_basis, plan.ch_in, plan.ch_out
    M3 = sum(2 * l3 + 1 for _, _, l3, _ in paths)
    M1 = sum(2 * l1 + 1 for l1, _, _, _ in paths)
    nnz = sum(n for *_, n in paths)
    S = 4 * N * K * Ci * M3
    T = 4 * N * K * Co * M1
    Wb = plan.w_numel * xbytes
    x = N * plan.rows_in * Ci * xbytes
    go = 4 * N * plan.rows_out * Co
    graph = 4 * (N + 1) + 4 * E + 12 * N
    return {
        "stream_fwd": (E * Ci * (2 * nnz + 2 * K * M3), x + graph + S),
        "stream_jvp": (E * Ci * (4 * nnz + 4 * K * M3), x + graph + 12 * N + S),
        "stream_snd": (E * Co * (2 * nnz + 2 * K * M1), go + graph + T),
        "stream_sndt": (E * Co * (4 * nnz + 4 * K * M1), go + graph + 12 * N + T),
        "stream_bwdpos": (E * Ci * (4 * nnz + 4 * K * M3), x + graph + S + 24 * N),
        "gemm_out": (2 * N * K * Ci * Co * M3, S + Wb + go),
        "gemm_gs": (2 * N * K * Ci * Co * M3, go + Wb + S),
        "gemm_gx": (2 * N * K * Ci * Co * M1, T + Wb + x // xbytes * 4),
        "gemm_gw": (2 * N * K * Ci * Co * M3, S + go + 4 * plan.w_numel),
        # channel-wise contractions (out side shown; the input side is the same size for these path sets)
        "cw_contract": (2 * N * K * Ci * M3, S + Wb + go),
        "cw_gw": (2 * N * K * Ci * M3, S + go),
    }


def roofline_for(name, flops, nbytes, ms):
    sec = ms * 1e-3
    t_alu = flops / (PEAK["alu"][0] * 1e12)
    t_hbm = nbytes / (PEAK["hbm"][0] * 1e9)
    if name.startswith("gemm"):
        bound = "mfma" if flops / (PEAK["mfma"][0] * 1e12) >= t_hbm else "hbm"
    else:
        bound = "alu" if t_alu >= t_hbm else "hbm"
    if bound == "hbm":
        achieved = nbytes / sec / 1e9
    else:
        achieved = flops / sec / 1e12
    peak, unit = PEAK[bound]
    return {"kernel": name, "bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "algorithmic_flops": int(flops), "algorithmic_bytes": int(nbytes),
            "avg_launch_us": round(ms * 1e3, 2)}


def load_traffic(workload, kernel):
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    from equivariant_gnn_tensor_receiver_amd.profiling import kernel_source_hash

    if t.get("source_hash") != kernel_source_hash():
        return None  # the kernel changed since the counters were taken
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(name, w, data, plan, sample_edges):
    """The fp64 oracle (materialising schedule) on the in-edges of the first receivers."""
    import numpy as np
    from oracle import tpconv as otp

    try:
        from threadpoolctl import threadpool_info

        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = 1
    prob = otp.Problem(w.irreps, w.irreps, w.lmax, w.num_basis, channelwise=w.channelwise)
    rowptr = data["rowptr"]
    nrecv = int(np.searchsorted(rowptr, sample_edges, side="right") - 1)
    nrecv = max(1, min(nrecv, w.num_nodes))
    e1 = int(rowptr[nrecv])
    snd = data["senders"][:e1].astype(np.int64)
    rcv = np.repeat(np.arange(nrecv), np.diff(rowptr[:nrecv + 1]))
    # repeated (whole passes) until about 10 s of CPU work when the sample is the whole graph
    reps, dt = 0, 0.0
    while reps == 0 or dt < 10.0:
        t0 = time.perf_counter()
        otp.forward(prob, data["pos"], snd, rcv, data["x"], data["W"], num_nodes=w.num_nodes)
        if "bwd" in w.passes:
            otp.backward(prob, data["pos"], snd, rcv, data["x"], data["W"], data["g_out"])
        if "dbwd" in w.passes:
            otp.double_backward(prob, data["pos"], snd, rcv, data["x"], data["W"], data["g_out"], data["gg_pos"])
        dt += time.perf_counter() - t0
        reps += 1
    passes = "+".join(p for p in w.passes)
    rep = f" x {reps} repetitions" if reps > 1 else ""
    return {"value": round(reps * e1 / dt, 2), "unit": "edges/s", "cores": int(cores), "kind": "oracle",
            "sample": f"in-edges of receivers 0..{nrecv - 1} ({e1} of {len(data['senders'])} edges){rep}, "
                      f"{passes}, fp64 numpy, {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="molecular")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-edges", type=int, default=0, help="oracle sample size (edges); 0 = default")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the path runs on a single "
              "MI355X; sharding over several GPUs is not built)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from equivariant_gnn_tensor_receiver_amd import inputs
    from equivariant_gnn_tensor_receiver_amd import tpconv as tp

    w = inputs.WORKLOADS[args.workload]
    dt_code = tp.TPCONV_BF16 if w.dtype == "bf16" else tp.TPCONV_F32
    plan = tp.Plan(w.irreps, w.irreps, w.lmax, w.num_basis, inputs.CUTOFF, 6, dt_code, dt_code,
                   tp.CHANNELWISE if w.channelwise else tp.FULLY_CONNECTED)
    t0 = time.perf_counter()
    data = inputs.make_workload(args.workload, plan.num_paths)
    t_gen = time.perf_counter() - t0
    N, E = w.num_nodes, len(data["senders"])
    dev = torch.device("cuda:0")
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    pos, rowptr, senders = to(data["pos"]), to(data["rowptr"]), to(data["senders"])
    if w.dtype == "bf16":
        x, W = tp.to_device_bf16(data["x"], dev), tp.to_device_bf16(data["W"], dev)
    else:
        x, W = to(data["x"]), to(data["W"])
    g_out, gg = to(data["g_out"]), to(data["gg_pos"])
    torch.cuda.synchronize()
    base_alloc = torch.cuda.memory_allocated()

    t0 = time.perf_counter()
    graph = tp.tpconv_graph_prepare(plan, tp.Graph(rowptr, senders), validate=True)
    torch.cuda.synchronize()
    t_prep = time.perf_counter() - t0

    f32 = dict(dtype=torch.float32, device=dev)
    out = torch.empty((N, plan.rows_out, plan.ch_out), **f32)
    S = torch.empty(plan.state_size(N) // 4, **f32)
    gx = torch.empty((N, plan.rows_in, plan.ch_in), **f32)
    gW = torch.empty(plan.w_shape, **f32)
    gp = torch.empty((N, 3), **f32)
    dW = torch.empty(plan.w_shape, **f32)
    dx = torch.empty((N, plan.rows_in, plan.ch_in), **f32)
    ws_b = torch.empty(plan.workspace_size(tp.OP_BACKWARD, N, E), dtype=torch.uint8, device=dev)
    ws_d = torch.empty(plan.workspace_size(tp.OP_DOUBLE_BACKWARD, N, E), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    io_alloc = torch.cuda.memory_allocated()

    def fwd():
        tp.tpconv_forward(plan, graph, pos, x, W, out=out, saved_state=S)

    def bwd():
        if args.workload == "force":
            tp.tpconv_backward(plan, graph, pos, x, W, g_out, saved_state=S, want=("pos",), workspace=ws_b,
                               grad_pos=gp)
        else:
            tp.tpconv_backward(plan, graph, pos, x, W, g_out, saved_state=S, workspace=ws_b, grad_x=gx,
                               grad_W=gW, grad_pos=gp)

    def dbwd():
        tp.tpconv_double_backward(plan, graph, pos, x, W, g_out, gg, want=("W", "x"), workspace=ws_d, d_W=dW,
                                  d_x=dx)

    step_parts = [fwd] + ([bwd] if "bwd" in w.passes else []) + ([dbwd] if "dbwd" in w.passes else [])

    def step():
        for f in step_parts:
            f()

    def timed(fn, k):
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(k):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t) / k * 1e3

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    ms_step = timed(step, args.steps)
    peak_alloc = torch.cuda.max_memory_allocated()
    value = E / (ms_step * 1e-3)

    passes = {}
    ms_f = timed(fwd, args.steps)
    passes["fwd"] = {"ms": round(ms_f, 4), "edges_per_s": round(E / (ms_f * 1e-3), 1)}
    if "bwd" in w.passes:
        ms_b = timed(bwd, args.steps)
        passes["bwd"] = {"ms": round(ms_b, 4)}
        passes["fwd+bwd"] = {"ms": round(ms_f + ms_b, 4), "edges_per_s": round(E / ((ms_f + ms_b) * 1e-3), 1)}
    if "dbwd" in w.passes:
        ms_d = timed(dbwd, args.steps)
        passes["dbwd"] = {"ms": round(ms_d, 4), "edges_per_s": round(E / (ms_d * 1e-3), 1)}

    # per-kernel HIP-event durations over a second timed region
    tp.tpconv_kernel_timing(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ktimes = tp.tpconv_kernel_timing_read()
    tp.tpconv_kernel_timing(False)
    xbytes = 2 if w.dtype == "bf16" else 4
    alg = algorithmic(plan, plan_counts(plan), N, E, xbytes)
    kernels = {}
    for name, (n, ms) in ktimes.items():
        kernels[name] = {"launches_per_step": n / args.steps, "avg_us": round(ms / n * 1e3, 2),
                         "share": round(ms / sum(v[1] for v in ktimes.values()), 4)}
    dom = max((k for k in ktimes if k in alg), key=lambda k: ktimes[k][1])
    n_dom, ms_dom = ktimes[dom]
    roof = roofline_for(dom, alg[dom][0], alg[dom][1], ms_dom / n_dom)
    roof["traffic"] = load_traffic(args.workload, dom)

    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "edges/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if w.dtype == "f32" else "bf16-in/f32",
        "data": "synthetic",
        "config": {"workload": w.name, "num_nodes": N, "num_edges": E, "mean_degree": round(E / N, 2),
                   "irreps": w.irreps, "sh_lmax": w.lmax, "num_basis": w.num_basis, "paths": plan.num_paths,
                   "step": "+".join(w.passes), "cutoff": inputs.CUTOFF, "box": round(data["box"], 4),
                   "connection": "channelwise" if w.channelwise else "fully_connected"},
        "passes": passes,
        "peak_bytes": {"workspace_fwd": plan.workspace_size(tp.OP_FORWARD, N, E),
                       "workspace_bwd": plan.workspace_size(tp.OP_BACKWARD, N, E),
                       "workspace_dbwd": plan.workspace_size(tp.OP_DOUBLE_BACKWARD, N, E),
                       "saved_state": plan.state_size(N),
                       "allocated_over_inputs": int(peak_alloc - base_alloc),
                       "allocated_over_inputs_outputs_ws": int(peak_alloc - io_alloc),
                       "csc_index": 4 * (N + 1 + E),
                       "conventional_edge_weights": 4 * E * plan.w_numel // plan.num_basis},
        "roofline": roof,
        "kernels": kernels,
        "setup_s": {"inputs": round(t_gen, 2), "graph_prepare": round(t_prep, 4)},
    }
    if not args.no_cpu_baseline:
        # about 10-30 s of oracle work on the host cores
        sample = args.cpu_sample_edges or {"tiny": 512, "molecular": 80000, "wide_l": 4000,
                                           "edge_scaling": 80000, "force": 2000,
                                           "molecular_uvu": 120000}[w.name]
        res["cpu_baseline"] = cpu_baseline(w.name, w, data, plan, sample)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
