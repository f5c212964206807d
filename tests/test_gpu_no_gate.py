"""GPU parity of the row-layout output kernels with the gate absent: y = C h + D x with no
SiLU(z) factor (page-3 report, section 3: the selective scan's output before the
MambaBlock multiplies it by SiLU of the gate branch).

For N = 16 the output kernels are compiled once with the gate present and once with it
absent (no z loads, no SiLU factor); the gate-absent case in test_gpu_parity runs 70
steps, too few to reach the kernels' steady loop.  These cases run several hundred
steps with a ragged last chunk through every gate-absent form: zero-order hold and
Euler, unsplit and as the main pass of the two-level split, with checkpoints, with the
convolution prologue, and with the structured-A staging.  Tolerance as in
test_gpu_parity.
"""
import numpy as np
import pytest

import workloads as W
from test_gpu_parity import TAU, assert_close, check_workload, f32dev, host, note, orc, ss, tdev  # noqa: F401

pytestmark = pytest.mark.gpu


def inputs(dtype, seed, batch=2, seqlen=603, dim=128):
    return W.make_scan_inputs(batch, seqlen, dim, 16, dtype, seed=seed, with_z=False, name="no gate")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("euler", [False, True])
@pytest.mark.parametrize("segs", [1, 3, None])
def test_no_gate_forward(ss, orc, dtype, euler, segs):
    w = inputs(dtype, 700 + 2 * euler + (segs or 0))
    check_workload(ss, orc, w, num_segments=segs, euler=euler,
                   label=f"no gate {dtype} euler={euler} segments={segs}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("euler", [False, True])
def test_no_gate_with_checkpoints(ss, orc, dtype, euler):
    import torch
    w = inputs(dtype, 710 + euler)
    note(f"[case] no gate with checkpoints {dtype} euler={euler}: B={w.batch} L={w.seqlen} D={w.dim}")
    x, dt, B, C = (tdev(a, dtype) for a in (w.x, w.dt, w.B, w.C))
    A, D, bias = f32dev(w.A), f32dev(w.D), f32dev(w.dt_bias)
    ck = torch.empty(ss.checkpoint_bytes(w.batch, w.seqlen, w.dim, w.dstate) // 4, dtype=torch.float32,
                     device="cuda")
    y = torch.full_like(x, float("nan"))
    y_plain = torch.full_like(x, float("nan"))
    ss.sscan_fwd(x, dt, A, B, C, D=D, delta_bias=bias, out=y, euler=euler, checkpoints=ck)
    ss.sscan_fwd(x, dt, A, B, C, D=D, delta_bias=bias, out=y_plain, euler=euler)
    torch.cuda.synchronize()
    yr, _ = orc.sscan_fwd(w.x, w.dt, w.A, w.B, w.C, D=w.D, z=None, dt_bias=w.dt_bias, euler=euler)
    e = assert_close(host(y), yr, TAU[dtype], "y")
    assert torch.equal(y, y_plain), "y with checkpoints differs from y without"
    note(f"       max rel err y={e:.3e}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_no_gate_conv_prologue(ss, orc, dtype):
    w = inputs(dtype, 720)
    K = 4
    rng = np.random.default_rng(721)
    cw = (0.5 * rng.standard_normal((w.dim, K))).astype(np.float32)
    cb = (0.1 * rng.standard_normal(w.dim)).astype(np.float32)
    note(f"[case] no gate, conv prologue {dtype}: B={w.batch} L={w.seqlen} D={w.dim} K={K}")
    y, st = ss.sscan_fwd(tdev(w.x, dtype), tdev(w.dt, dtype), f32dev(w.A), tdev(w.B, dtype), tdev(w.C, dtype),
                         D=f32dev(w.D), delta_bias=f32dev(w.dt_bias), return_last_state=True,
                         conv_w=f32dev(cw), conv_b=f32dev(cb))
    u, _ = orc.conv_silu_prologue(w.x, cw, cb)
    yr, sr = orc.sscan_fwd(u, w.dt, w.A, w.B, w.C, D=w.D, z=None, dt_bias=w.dt_bias)
    assert_close(host(y), yr, TAU[dtype], "y")
    assert_close(host(st), sr, TAU[dtype], "last_state")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_no_gate_structured(ss, orc, dtype):
    import torch
    w = inputs(dtype, 730)
    note(f"[case] no gate, structured A {dtype}: B={w.batch} L={w.seqlen} D={w.dim}")
    x, dt, B, C = (tdev(a, dtype) for a in (w.x, w.dt, w.B, w.C))
    y = torch.full_like(x, float("nan"))
    st = torch.full((w.batch, w.dim, w.dstate), float("nan"), dtype=torch.float32, device="cuda")
    ss.sscan_fwd(x, dt, f32dev(w.A), B, C, D=f32dev(w.D), delta_bias=f32dev(w.dt_bias), out=y, last_state=st,
                 structured_a=True)
    torch.cuda.synchronize()
    yr, sr = orc.sscan_fwd(w.x, w.dt, w.A, w.B, w.C, D=w.D, z=None, dt_bias=w.dt_bias)
    assert_close(host(y), yr, TAU[dtype], "y")
    assert_close(host(st), sr, TAU[dtype], "last_state")
