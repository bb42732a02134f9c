"""Deterministic position gradients (plans created with deterministic=True):
grad_pos and d_pos are sums of per-edge shares added as exact 64-bit fixed
point, so they are bitwise the same whatever order the streams visit the
nodes in (here: index order against the Morton order, and repeated runs),
and they still match the fp64 oracle."""
import numpy as np
import pytest

from gpu_cases import GRAD_TOL, DeviceCase, rel_err, say
from equivariant_gnn_tensor_receiver_amd import inputs
from equivariant_gnn_tensor_receiver_amd import tpconv as tp

pytestmark = pytest.mark.gpu

CASES = [
    # name, irreps_in, irreps_out, sh_lmax, K, N, deg, x dtype, options
    ("det_l2_c32", "32x0e+32x1o+32x2e", "32x0e+32x1o+32x2e", 2, 8, 300, 40, "f32", {}),
    ("det_mixed_k16", "16x0e+16x1o+16x1e+16x2e", "8x0e+8x0o+8x1o+8x1e+8x2e+8x3o", 2, 16, 120, 30, "f32", {}),
    ("det_l3_bf16", "16x0e+16x1o+16x2e+16x3o", "16x0e+16x1o+16x2e+16x3o", 3, 8, 100, 30, "bf16", {}),
    ("det_channelwise", "32x0e+32x1o+32x2e", "32x0e+32x1o+32x2e", 2, 8, 200, 40, "f32", dict(channelwise=True)),
    ("det_radial_mlp", "16x0e+16x1o+16x2e", "16x0e+16x1o+16x2e", 2, 8, 150, 30, "f32", dict(radial_mlp=True)),
]


def pair(spec):
    name, ii, io, lsh, K, N, deg, dt, opt = spec
    graph = inputs.random_graph(N, deg, seed=7)
    a = DeviceCase(ii, io, lsh, K, *graph, dtype=dt, ordered=False, deterministic=True, **opt)
    b = DeviceCase(ii, io, lsh, K, *inputs.random_graph(N, deg, seed=7), dtype=dt, ordered=True, deterministic=True,
                   **opt)
    return a, b


@pytest.mark.parametrize("spec", CASES, ids=[c[0] for c in CASES])
def test_deterministic_position_gradients(spec):
    say(f"[case] {spec[0]}: deterministic grad_pos and d_pos, index order against Morton order")
    a, b = pair(spec)
    gp_a = a.backward(want=("pos",))[2]
    gp_b = b.backward(want=("pos",))[2]
    gp_a2 = a.backward(want=("pos",))[2]
    assert np.array_equal(gp_a, gp_b) and np.array_equal(gp_a, gp_a2)
    ref = a.o_backward(a.np["g_out"])[2]
    e = rel_err(gp_a, ref)
    say(f"  g_pos rel err {e:.2e}")
    assert e <= GRAD_TOL
    dp_a = a.double_backward(want=("pos",))[3]
    dp_b = b.double_backward(want=("pos",))[3]
    assert np.array_equal(dp_a, dp_b)
    e = rel_err(dp_a, a.o_double_backward(a.np["g_out"])[3])
    say(f"  d_pos rel err {e:.2e}")
    assert e <= GRAD_TOL


@pytest.mark.slow
@pytest.mark.parametrize("name", ["molecular", "edge_scaling"])
def test_deterministic_full_size(name):
    say(f"[workload] {name}, deterministic grad_pos in index and Morton order")
    w = inputs.WORKLOADS[name]
    pos, rowptr, senders, _, rng = inputs.make_graph(w)
    a = DeviceCase(w.irreps, w.irreps, w.lmax, w.num_basis, pos, rowptr, senders, rng, w.dtype, ordered=False,
                   deterministic=True)
    b = DeviceCase(w.irreps, w.irreps, w.lmax, w.num_basis, pos, rowptr, senders,
                   np.random.default_rng(0), w.dtype, ordered=True, deterministic=True)
    b.x, b.W, b.g_out = a.x, a.W, a.g_out  # the same inputs in both
    ga = a.backward(want=("pos",))[2]
    gb = b.backward(want=("pos",))[2]
    assert np.array_equal(ga, gb)
    plain = DeviceCase(w.irreps, w.irreps, w.lmax, w.num_basis, pos, rowptr, senders, np.random.default_rng(0),
                       w.dtype, ordered=True)
    plain.x, plain.W, plain.g_out = a.x, a.W, a.g_out
    gp = plain.backward(want=("pos",))[2]
    e = rel_err(gp, ga)
    say(f"  fp32-atomic against fixed-point grad_pos: {e:.2e}")
    assert e <= 1e-5
