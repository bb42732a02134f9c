"""The allocation-free forward (tpconv_forward_static) against tpconv_forward.

tpconv_forward_static keeps the receiver state in the library's static
per-device scratch instead of caller workspace.  Two calls in a row, the
second on a smaller graph, must each match tpconv_forward on the same inputs
(the same kernels run, so the results are identical), allocate nothing, and a
problem whose state exceeds the scratch is refused before any launch.
"""
import numpy as np
import pytest

from gpu_cases import FWD_TOL, rel_err, say
from equivariant_gnn_tensor_receiver_amd import inputs
from equivariant_gnn_tensor_receiver_amd import tpconv as tp

pytestmark = pytest.mark.gpu

IRREPS = "32x0e+32x1o+32x2e"


def upload(plan, N, deg, seed):
    import torch

    pos, rowptr, senders, rng = inputs.random_graph(N, deg, seed)
    t = inputs.make_tensors(rng, N, plan.rows_in, plan.ch_in, plan.rows_out, plan.ch_out, plan.num_basis,
                            plan.num_paths)
    dev = torch.device("cuda:0")
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    graph = tp.Graph(to(rowptr), to(senders))
    return graph, to(pos), to(t["x"]), to(t["W"])


def test_static_forward_matches_forward_twice():
    import torch

    plan = tp.Plan(IRREPS, IRREPS, 2, 8)
    assert plan.workspace_size(tp.OP_FORWARD, 1700, 0) <= tp.STATIC_SCRATCH_BYTES
    for call, (N, deg, seed) in enumerate(((1700, 24, 7), (300, 12, 8))):
        say(f"[case] static-scratch forward, call {call + 1}: N={N} deg~{deg}")
        graph, pos, x, W = upload(plan, N, deg, seed)
        ref = tp.tpconv_forward(plan, graph, pos, x, W)
        out = torch.full_like(ref, float("nan"))
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        tp.tpconv_forward_static(plan, graph, pos, x, W, out)
        torch.cuda.synchronize()
        assert torch.cuda.max_memory_allocated() == base
        a, b = out.cpu().numpy(), ref.cpu().numpy()
        e = rel_err(a, b)
        say(f"  rel err vs tpconv_forward {e:.2e}, identical {np.array_equal(a, b)}")
        assert e <= FWD_TOL
        assert np.array_equal(a, b)


def test_static_forward_refuses_oversize_problem():
    import torch

    plan = tp.Plan(IRREPS, IRREPS, 2, 8)
    N = tp.STATIC_SCRATCH_BYTES // (8 * 32 * 35 * 4) + 1
    dev = torch.device("cuda:0")
    rowptr = torch.zeros(N + 1, dtype=torch.int32, device=dev)
    senders = torch.zeros(1, dtype=torch.int32, device=dev)
    g = tp.Graph(rowptr, senders)
    g.num_edges = 0
    pos = torch.zeros((N, 3), dtype=torch.float32, device=dev)
    x = torch.zeros((N, plan.rows_in, plan.ch_in), dtype=torch.float32, device=dev)
    W = torch.zeros(plan.w_shape, dtype=torch.float32, device=dev)
    out = torch.zeros((N, plan.rows_out, plan.ch_out), dtype=torch.float32, device=dev)
    with pytest.raises(tp.TpconvError) as e:
        tp.tpconv_forward_static(plan, g, pos, x, W, out)
    assert e.value.status == 7
