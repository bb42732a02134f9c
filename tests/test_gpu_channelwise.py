"""GPU parity of the channel-wise ("uvu") connection against the fp64 oracle.

Same streams as the fully connected operator; the contractions are the
channel-diagonal kernels and the position-gradient stream forms its cotangent
W[k, p, c] g_out in registers.  Cases cover natural and mixed irreps, K = 8
and 16, bf16 inputs, channel tiles of 4 to 64 and a channel count that is not
a multiple of 4.
"""
import zlib

import numpy as np
import pytest

from gpu_cases import FWD_TOL, GRAD_TOL, DeviceCase, rel_err, say
from equivariant_gnn_tensor_receiver_amd import inputs

pytestmark = pytest.mark.gpu

CASES = [
    # name, irreps_in, irreps_out, sh_lmax, K, N, deg, dtype
    ("cw_l2_c32", "32x0e+32x1o+32x2e", "32x0e+32x1o+32x2e", 2, 8, 150, 20, "f32"),
    ("cw_l2_c128_k16", "128x0e+128x1o+128x2e", "128x0e+128x1o+128x2e", 2, 16, 40, 14, "f32"),
    ("cw_l3_c16_bf16", "16x0e+16x1o+16x2e+16x3o", "16x0e+16x1o+16x2e+16x3o", 3, 8, 60, 14, "bf16"),
    ("cw_mixed", "8x0e+8x1o+8x1e+8x2e", "8x0e+8x0o+8x1o+8x1e+8x2e+8x3o", 2, 8, 50, 12, "f32"),
    ("cw_c3_k16", "3x0e+3x1o+3x2e", "3x0e+3x1o+3x2e", 2, 16, 40, 90, "f32"),
    ("cw_l3_k16", "16x0e+16x1o+16x2e+16x3o", "16x0e+16x1o+16x2e+16x3o", 3, 16, 30, 40, "f32"),
    # an output irrep (2o) that no path reaches and an input irrep (3o) that reaches nothing
    ("cw_no_path_groups", "8x0e+8x1o+8x3o", "8x0e+8x1o+8x2o", 1, 8, 50, 12, "f32"),
    # ragged multiplicities: each path joins irreps of equal channel counts
    ("cw_ragged", "16x0e+8x1e+12x2e", "16x0e+8x1e+12x2e", 1, 8, 50, 12, "f32"),
]


@pytest.fixture(scope="module", params=CASES, ids=[c[0] for c in CASES])
def case(request):
    name, ii, io, lsh, K, N, deg, dt = request.param
    say(f"[case] {name}: N={N} deg~{deg} irreps_in={ii} irreps_out={io} lsh={lsh} K={K} {dt} channel-wise")
    seed = zlib.crc32(name.encode()) % 1000
    return DeviceCase(ii, io, lsh, K, *inputs.random_graph(N, deg, seed=seed), dtype=dt, channelwise=True)


def test_cw_forward(case):
    say("[step] forward")
    e = rel_err(case.forward(), case.o_forward())
    say(f"  fwd rel err {e:.2e}")
    assert e <= FWD_TOL


def test_cw_forward_saved_state_deterministic(case):
    import torch

    S = torch.empty(case.plan.state_size(case.graph.num_nodes) // 4, dtype=torch.float32, device=case.dev)
    assert np.array_equal(case.forward(saved_state=S), case.forward())


def test_cw_backward(case):
    say("[step] backward")
    gx, gW, gp = case.backward()
    rx, rW, rp = case.o_backward(case.np["g_out"])
    ex, eW, ep = rel_err(gx, rx), rel_err(gW, rW), rel_err(gp, rp)
    say(f"  g_x {ex:.2e}  g_W {eW:.2e}  g_pos {ep:.2e}")
    assert ex <= GRAD_TOL and eW <= GRAD_TOL and ep <= GRAD_TOL


def test_cw_double_backward(case):
    say("[step] double backward")
    dW, dx, dgo, dp = case.double_backward()
    rW, rx, rgo, rp = case.o_double_backward(case.np["g_out"])
    eW, ex, eg, ep = rel_err(dW, rW), rel_err(dx, rx), rel_err(dgo, rgo), rel_err(dp, rp)
    say(f"  d_W {eW:.2e}  d_x {ex:.2e}  d_g_out {eg:.2e}  d_pos {ep:.2e}")
    assert eW <= GRAD_TOL and ex <= GRAD_TOL and eg <= GRAD_TOL and ep <= GRAD_TOL
