#!/usr/bin/env python3
"""Throughput of the streaming CG tensor-product convolution on one MI355X.

A step is one pass of the workload's hot path over its synthetic radius graph:
forward (receiver stream + contraction) and backward w.r.t. x, W and
positions; the "force" workload runs forward, the position gradient (forces)
and the double backward of the force loss.  Inputs are resident in HBM before
the timed region.

Prints ONE JSON line.  `value` is edges/s of the headline workload's step
(Edge-scaling by default, the largest configuration).  The line also carries,
for that workload, per-pass throughput, peak workspace bytes, the dominant
kernel's roofline (algorithmic FLOPs or bytes per launch over its HIP-event
duration) and the CPU oracle's throughput on a bounded sample; and under
`per_config`, every configuration's forward and fwd+bwd (Force: each stage of
its chain) edges/s with the whole-pass lower bound T_lb and T_lb / T_measured,
and Molecular once more with the radial MLP in front of the streams
(`molecular_radial_mlp`, its backward including the MLP's weight gradient).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload edge_scaling]
       [--no-all-configs] [--no-cpu-baseline] [--radial-mlp (with --no-cpu-baseline: the
       named workload alone, with the radial MLP)]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "edges/sec fwd and fwd+bwd per config; % of HBM/MFMA roofline; peak bytes"
HBM_GBS = 8000.0          # MI355X HBM3E
FP32_TFLOPS = 157.3       # fp32 MFMA, and packed fp32 VALU (256 CUs x 4 SIMDs x 64 FLOP/clk x 2.4 GHz)
BF16_TFLOPS = 2500.0      # dense bf16 MFMA
PEAK = {"hbm": (HBM_GBS, "GB/s"), "alu": (FP32_TFLOPS, "TFLOP/s")}


def gemm_peak(name, w_bf16):
    """Peak of an fp32-accurate contraction on the bf16 matrix cores: each fp32
    operand is split into bf16 hi + lo, so one product takes three bf16
    products (two when the weights are bf16 already; gW multiplies two fp32
    operands either way)."""
    return BF16_TFLOPS / (2 if w_bf16 and name != "gemm_gw" else 3)
CONFIG_ORDER = ("tiny", "molecular", "wide_l", "edge_scaling", "force", "molecular_uvu")


def plan_counts(plan):
    """Per-path (l1, l2, l3, nnz) from the plan's own tables."""
    import numpy as np

    out = []
    for i in range(plan.num_paths):
        (l1, l2, l3), _ = plan.path(i)
        out.append((l1, l2, l3, int((np.abs(plan.cg(i)) > 1e-12).sum())))
    return out


def sizes(plan, N, E, xbytes, wbytes):
    """Bytes of every tensor a pass must read or write once."""
    fin, fout, wf = 4 * N * plan.rows_in * plan.ch_in, 4 * N * plan.rows_out * plan.ch_out, 4 * plan.w_numel
    return {"x": N * plan.rows_in * plan.ch_in * xbytes, "W": plan.w_numel * wbytes, "pos": 12 * N,
            "csr": 4 * (N + 1) + 4 * E, "csc": 4 * (N + 1) + 4 * E, "out": fout, "g_out": fout, "g_x": fin,
            "gW": wf, "g_pos": 12 * N, "gg_pos": 12 * N, "d_W": wf, "d_x": fin, "d_g_out": fout,
            "d_pos": 12 * N}


def algorithmic(plan, paths, N, E, xbytes, wbytes):
    """Algorithmic FLOPs and compulsory HBM bytes per launch of each kernel class.

    Edge streams count the coupling (2 C nnz per edge and direction) and the
    radial products (2 K C M per edge and direction); the per-edge weights and
    messages of the conventional schedule are not counted.  A stream writes
    (or reads) its node-sized state once."""
    K, Ci, Co = plan.num_basis, plan.ch_in, plan.ch_out
    M3 = sum(2 * l3 + 1 for _, _, l3, _ in paths)
    M1 = sum(2 * l1 + 1 for l1, _, _, _ in paths)
    nnz = sum(n for *_, n in paths)
    S = 4 * N * K * Ci * M3
    T = 4 * N * K * Co * M1
    z = sizes(plan, N, E, xbytes, wbytes)
    x, Wb, go, graph = z["x"], z["W"], z["g_out"], z["csr"] + z["pos"]
    return {
        "stream_fwd": (E * Ci * (2 * nnz + 2 * K * M3), x + graph + S),
        "stream_jvp": (E * Ci * (4 * nnz + 4 * K * M3), x + graph + 12 * N + S),
        "stream_snd": (E * Co * (2 * nnz + 2 * K * M1), go + graph + T),
        "stream_sndt": (E * Co * (4 * nnz + 4 * K * M1), go + graph + 12 * N + T),
        "stream_bwdpos": (E * Ci * (4 * nnz + 4 * K * M3), x + graph + S + 12 * N),
        # Hessian term of dL/dpos: K-sums with R, R', R'' and three couplings
        "stream_hess": (E * Ci * (6 * nnz + 6 * K * M3), x + graph + S + 24 * N),
        "gemm_out": (2 * N * K * Ci * Co * M3, S + Wb + go),
        "gemm_gs": (2 * N * K * Ci * Co * M3, go + Wb + S),
        "gemm_gx": (2 * N * K * Ci * Co * M1, T + Wb + z["g_x"]),
        "gemm_gw": (2 * N * K * Ci * Co * M3, S + go + 4 * plan.w_numel),
        # channel-wise contractions (out side shown; the input side is the same size for these path sets)
        "cw_contract": (2 * N * K * Ci * M3, S + Wb + go),
        "cw_gw": (2 * N * K * Ci * M3, S + go),
    }


# Kernel classes of each pass and the tensors it must read or write once.
PASS_KERNELS = {
    "fwd": (("stream_fwd", "gemm_out"), {"x", "W", "pos", "csr", "out"}),
    # backward w.r.t. x, W and positions
    "bwd": (("stream_snd", "gemm_gx", "gemm_gw", "gemm_gs", "stream_bwdpos"),
            {"x", "W", "pos", "csr", "csc", "g_out", "g_x", "gW", "g_pos"}),
    # Force chain: the position gradient only, then the double backward w.r.t. W and x
    "forces": (("gemm_gs", "stream_bwdpos"), {"x", "W", "pos", "csr", "g_out", "g_pos"}),
    "dbwd": (("stream_jvp", "gemm_gw", "stream_sndt", "gemm_gx"),
             {"x", "W", "pos", "csr", "csc", "g_out", "gg_pos", "d_W", "d_x"}),
    # the whole double backward: also d_grad_out (S-dot W) and dL/dpos (gS, then the Hessian stream)
    "dbwd_all": (("stream_jvp", "gemm_gw", "stream_sndt", "gemm_gx", "gemm_out", "gemm_gs", "stream_hess"),
                 {"x", "W", "pos", "csr", "csc", "g_out", "gg_pos", "d_W", "d_x", "d_g_out", "d_pos"}),
}
CW_KERNEL = {"gemm_out": "cw_contract", "gemm_gx": "cw_contract", "gemm_gw": "cw_gw", "gemm_gs": None}


def pass_bound(names, alg, channelwise, w_bf16, nbytes):
    """T_lb = max(bytes / HBM, VALU FLOPs / VALU peak, contraction FLOPs / their peak), perfect overlap assumed."""
    valu = mfma = 0
    t_mfma = 0.0
    for n in names:
        if channelwise and n in CW_KERNEL:
            n = CW_KERNEL[n]
            if n is None:
                continue
            valu += alg[n][0]  # channel-diagonal contractions run on the vector ALUs
        elif n.startswith("gemm"):
            mfma += alg[n][0]
            t_mfma += alg[n][0] / (gemm_peak(n, w_bf16) * 1e12)
        else:
            valu += alg[n][0]
    terms = {"hbm": nbytes / (HBM_GBS * 1e9), "alu": valu / (FP32_TFLOPS * 1e12), "mfma": t_mfma}
    bind = max(terms, key=terms.get)
    return terms[bind], bind, valu, mfma


def roofline_for(name, flops, nbytes, ms, w_bf16):
    sec = ms * 1e-3
    t_alu = flops / (PEAK["alu"][0] * 1e12)
    t_hbm = nbytes / (PEAK["hbm"][0] * 1e9)
    if name.startswith("gemm"):
        bound = "mfma" if flops / (gemm_peak(name, w_bf16) * 1e12) >= t_hbm else "hbm"
    else:
        bound = "alu" if t_alu >= t_hbm else "hbm"
    if bound == "hbm":
        achieved = nbytes / sec / 1e9
    else:
        achieved = flops / sec / 1e12
    peak, unit = (round(gemm_peak(name, w_bf16), 1), "TFLOP/s") if bound == "mfma" else PEAK[bound]
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

    if t.get("source_hash") != kernel_source_hash(kernel):
        return None  # the kernel changed since the counters were taken
    return t.get("hbm_bytes_per_launch")


def host_info():
    """Cores this process may run on, the CPU model and numpy's BLAS."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas, threads = "unknown", 1
    try:
        from threadpoolctl import threadpool_info

        for i in threadpool_info():
            if i.get("user_api") == "blas":
                blas = f"{i.get('internal_api')} {i.get('version')}"
                threads = max(threads, int(i.get("num_threads", 1)))
    except Exception:  # pragma: no cover
        pass
    return {"affinity_cores": len(os.sched_getaffinity(0)), "cpu_model": model, "blas": blas,
            "blas_threads": threads}


def cpu_baseline(w, data, sample_edges):
    """The fp64 oracle (materialising schedule) on the in-edges of the first receivers."""
    import numpy as np
    from oracle import tpconv as otp

    host = host_info()
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
    # numpy's einsum contractions run on BLAS; its thread count is what the oracle used
    return {"value": round(reps * e1 / dt, 2), "unit": "edges/s", "cores": host["blas_threads"], "kind": "oracle",
            "sample": f"in-edges of receivers 0..{nrecv - 1} ({e1} of {len(data['senders'])} edges){rep}, "
                      f"{passes}, fp64 numpy, {dt:.1f} s",
            "host": host}


def run_workload(name, steps, warmup, detail, radial_mlp=False):
    """Time one workload; returns its report (and the oracle inputs when `detail`).

    radial_mlp: put the radial MLP (one SiLU layer K wide on the basis) in
    front of the streams; the backward and double backward then also return
    its weight gradient."""
    import numpy as np
    import torch

    from equivariant_gnn_tensor_receiver_amd import inputs
    from equivariant_gnn_tensor_receiver_amd import tpconv as tp

    w = inputs.WORKLOADS[name]
    dt_code = tp.TPCONV_BF16 if w.dtype == "bf16" else tp.TPCONV_F32
    plan = tp.Plan(w.irreps, w.irreps, w.lmax, w.num_basis, inputs.CUTOFF, 6, dt_code, dt_code,
                   tp.CHANNELWISE if w.channelwise else tp.FULLY_CONNECTED, radial_mlp)
    t0 = time.perf_counter()
    data = inputs.make_workload(name, plan.num_paths)
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
    K = w.num_basis
    mlp = {}
    if radial_mlp:
        A = np.random.default_rng(w.seed + 100).standard_normal((K, K)).astype(np.float32) * np.float32(1.5 / K ** 0.5)
        mlp = dict(radial_w=to(A), grad_radial_w=torch.empty((K, K), dtype=torch.float32, device=dev))
    mlp_fwd = {"radial_w": mlp["radial_w"]} if mlp else {}
    mlp_d = dict(radial_w=mlp["radial_w"], d_radial_w=torch.empty((K, K), dtype=torch.float32, device=dev)) if mlp else {}
    torch.cuda.synchronize()
    base_alloc = torch.cuda.memory_allocated()

    t0 = time.perf_counter()
    graph = tp.tpconv_graph_prepare(plan, tp.Graph(rowptr, senders), validate=True)
    graph = tp.tpconv_graph_order(plan, graph, pos)  # Morton visiting order of the nodes
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
    dg = torch.empty((N, plan.rows_out, plan.ch_out), **f32) if "dbwd" in w.passes else None
    dpos = torch.empty((N, 3), **f32)
    ws_f = torch.empty(max(1, plan.workspace_size(tp.OP_FORWARD_SAVED, N, E)), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(plan.workspace_size(tp.OP_BACKWARD, N, E), dtype=torch.uint8, device=dev)
    ws_d = torch.empty(plan.workspace_size(tp.OP_DOUBLE_BACKWARD, N, E), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    io_alloc = torch.cuda.memory_allocated()
    force = name == "force"

    def fwd():
        tp.tpconv_forward(plan, graph, pos, x, W, out=out, saved_state=S, workspace=ws_f, **mlp_fwd)

    def bwd():
        if force:  # forces: the position gradient only
            tp.tpconv_backward(plan, graph, pos, x, W, g_out, saved_state=S, want=("pos",), workspace=ws_b,
                               grad_pos=gp, **mlp)
        else:
            tp.tpconv_backward(plan, graph, pos, x, W, g_out, saved_state=S, workspace=ws_b, grad_x=gx,
                               grad_W=gW, grad_pos=gp, **mlp)

    def dbwd():
        tp.tpconv_double_backward(plan, graph, pos, x, W, g_out, gg, want=("W", "x"), workspace=ws_d, d_W=dW,
                                  d_x=dx, **mlp_d)

    def dbwd_all():
        tp.tpconv_double_backward(plan, graph, pos, x, W, g_out, gg, want=("W", "x", "grad_out", "pos"),
                                  workspace=ws_d, d_W=dW, d_x=dx, d_grad_out=dg, d_pos=dpos, **mlp_d)

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

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    ms_step = timed(step, steps)
    peak_alloc = torch.cuda.max_memory_allocated()

    xbytes = wbytes = 2 if w.dtype == "bf16" else 4
    alg = algorithmic(plan, plan_counts(plan), N, E, xbytes, wbytes)
    z = sizes(plan, N, E, xbytes, wbytes)
    w_bf16 = w.dtype == "bf16"

    def bound(pass_names, measured_ms):
        ks, ts = [], set()
        for pn in pass_names:
            ks += PASS_KERNELS[pn][0]
            ts |= PASS_KERNELS[pn][1]  # a tensor several passes of one step touch counts once
        nbytes = sum(z[t] for t in ts)
        t_lb, bind, valu, mfma = pass_bound(ks, alg, w.channelwise, w_bf16, nbytes)
        return {"ms": round(measured_ms, 4), "edges_per_s": round(E / (measured_ms * 1e-3), 1),
                "t_lb_us": round(t_lb * 1e6, 2), "binding": bind, "frac_of_bound": round(t_lb / (measured_ms * 1e-3), 4),
                "valu_gflop": round(valu / 1e9, 3), "mfma_gflop": round(mfma / 1e9, 3),
                "compulsory_mb": round(nbytes / 1e6, 2)}

    passes = {}
    ms_f = timed(fwd, steps)
    passes["fwd"] = bound(["fwd"], ms_f)
    if "bwd" in w.passes:
        ms_b = timed(bwd, steps)
        key = "forces" if force else "bwd"
        passes[key] = bound([key], ms_b)
        passes["fwd+" + key] = bound(["fwd", key], ms_f + ms_b)
    if "dbwd" in w.passes:
        ms_d = timed(dbwd, steps)
        passes["dbwd"] = bound(["dbwd"], ms_d)
        passes["fwd+forces+dbwd"] = bound(["fwd", "forces", "dbwd"], ms_f + ms_b + ms_d)
        passes["dbwd_all"] = bound(["dbwd_all"], timed(dbwd_all, steps))

    rep = {"workload": w.name, "num_nodes": N, "num_edges": E, "step": "+".join(w.passes),
           "ms_per_step": round(ms_step, 4), "edges_per_s": round(E / (ms_step * 1e-3), 1), "passes": passes}
    if not detail:
        return rep, None

    # per-kernel HIP-event durations over a second timed region
    tp.tpconv_kernel_timing(True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ktimes = tp.tpconv_kernel_timing_read()
    tp.tpconv_kernel_timing(False)
    kernels = {}
    for kname, (n, ms) in ktimes.items():
        kernels[kname] = {"launches_per_step": n / steps, "avg_us": round(ms / n * 1e3, 2),
                          "share": round(ms / sum(v[1] for v in ktimes.values()), 4)}
    dom = max((k for k in ktimes if k in alg), key=lambda k: ktimes[k][1])
    n_dom, ms_dom = ktimes[dom]
    roof = roofline_for(dom, alg[dom][0], alg[dom][1], ms_dom / n_dom, w_bf16)
    # the counter files are taken on the plain layer
    roof["traffic"] = None if radial_mlp else load_traffic(w.name, dom)
    rep.update({
        "value": E / (ms_step * 1e-3),
        "dtype": "f32" if w.dtype == "f32" else "bf16-in/f32",
        "config": {"workload": w.name, "num_nodes": N, "num_edges": E, "mean_degree": round(E / N, 2),
                   "irreps": w.irreps, "sh_lmax": w.lmax, "num_basis": w.num_basis, "paths": plan.num_paths,
                   "step": "+".join(w.passes), "cutoff": inputs.CUTOFF, "box": round(data["box"], 4),
                   "connection": "channelwise" if w.channelwise else "fully_connected",
                   **({"radial_mlp": True} if radial_mlp else {})},
        "peak_bytes": {"workspace_fwd": plan.workspace_size(tp.OP_FORWARD, N, E),
                       "workspace_fwd_saved": plan.workspace_size(tp.OP_FORWARD_SAVED, N, E),
                       "workspace_bwd": plan.workspace_size(tp.OP_BACKWARD, N, E),
                       "workspace_dbwd": plan.workspace_size(tp.OP_DOUBLE_BACKWARD, N, E),
                       "saved_state": plan.state_size(N),
                       "allocated_over_inputs": int(peak_alloc - base_alloc),
                       "allocated_over_inputs_outputs_ws": int(peak_alloc - io_alloc),
                       "csc_index": 4 * (N + 1 + E),
                       "conventional_edge_weights": 4 * E * plan.w_numel // plan.num_basis},
        "roofline": roof, "kernels": kernels,
        "setup_s": {"inputs": round(t_gen, 2), "graph_prepare": round(t_prep, 4)},
    })
    return rep, (w, data)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="edge_scaling")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-all-configs", action="store_true", help="time the headline workload only")
    ap.add_argument("--cpu-sample-edges", type=int, default=0, help="oracle sample size (edges); 0 = default")
    ap.add_argument("--radial-mlp", action="store_true",
                    help="time the headline workload with the radial MLP (needs --no-cpu-baseline)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the path runs on a single "
              "MI355X; sharding over several GPUs is not built)", file=sys.stderr)
        sys.exit(2)

    if args.radial_mlp and not args.no_cpu_baseline:
        print("--radial-mlp times the MLP variant only; the oracle baseline is the plain layer: add "
              "--no-cpu-baseline", file=sys.stderr)
        sys.exit(2)

    import torch

    head, oracle_inputs = run_workload(args.workload, args.steps, args.warmup, detail=True,
                                       radial_mlp=args.radial_mlp)
    per_config = {}
    if not args.no_all_configs and not args.radial_mlp:
        for name in CONFIG_ORDER:
            if name == args.workload:
                per_config[name] = {k: head[k] for k in ("num_edges", "step", "ms_per_step", "edges_per_s",
                                                         "passes")}
                continue
            torch.cuda.empty_cache()
            rep, _ = run_workload(name, max(5, args.steps // 2), 2, detail=False)
            per_config[name] = {k: rep[k] for k in ("num_edges", "step", "ms_per_step", "edges_per_s", "passes")}
            print(f"[bench] {name}: {rep['ms_per_step']:.4f} ms/step", file=sys.stderr, flush=True)
        # Molecular with the radial MLP in front of the streams (its backward
        # also returns the MLP's weight gradient: K more receiver-stream
        # passes); the bounds in `passes` are those of the plain layer
        torch.cuda.empty_cache()
        rep, _ = run_workload("molecular", max(5, args.steps // 2), 2, detail=False, radial_mlp=True)
        per_config["molecular_radial_mlp"] = {k: rep[k] for k in ("num_edges", "step", "ms_per_step", "edges_per_s",
                                                                  "passes")}
        print(f"[bench] molecular_radial_mlp: {rep['ms_per_step']:.4f} ms/step", file=sys.stderr, flush=True)

    res = {
        "metric": METRIC,
        "value": round(head["value"], 1),
        "unit": "edges/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic",
        "config": head["config"],
        "passes": head["passes"],
        "peak_bytes": head["peak_bytes"],
        "roofline": head["roofline"],
        "kernels": head["kernels"],
        "setup_s": head["setup_s"],
        "per_config": per_config,
    }
    if not args.no_cpu_baseline:
        w, data = oracle_inputs
        # about 10-30 s of oracle work on the host cores
        sample = args.cpu_sample_edges or {"tiny": 512, "molecular": 80000, "wide_l": 4000,
                                           "edge_scaling": 80000, "force": 2000,
                                           "molecular_uvu": 120000}[w.name]
        res["cpu_baseline"] = cpu_baseline(w, data, sample)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
