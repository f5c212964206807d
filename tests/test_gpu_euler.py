"""GPU parity of the Euler variant (Bbar = Delta B, the first-order rule of the page-3
report's code, section 4.2) against the oracle's Euler variant, same tolerances as
the zero-order-hold path."""
import numpy as np
import pytest

import workloads as W
from test_gpu_parity import (TAU, assert_close, check_workload, f32dev, host, note, orc, ss,  # noqa: F401
                             tdev)

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(600)
def test_euler_mamba130m_layer(ss, orc):
    w = W.workload("mamba130m_layer")
    check_workload(ss, orc, w, euler=True, label="mamba130m_layer Euler, auto segments")


@pytest.mark.timeout(900)
def test_euler_train_shape(ss, orc):
    check_workload(ss, orc, W.workload("train_shape"), euler=True, label="train_shape Euler")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [1, 3, 8, 13, 16])
def test_euler_ragged(ss, orc, dtype, N):
    w = W.make_scan_inputs(2, 53, 100, N, dtype, seed=300 + N, name=f"Euler ragged N={N}")
    check_workload(ss, orc, w, euler=True)


@pytest.mark.parametrize("segs", [1, 3])
def test_euler_segments_initial_state_zero_A(ss, orc, segs):
    w = W.make_scan_inputs(2, 300, 130, 16, "f32", seed=301, name="Euler segments")
    w.A = w.A.copy()
    w.A[3, :] = 0.0
    h0 = np.random.default_rng(5).standard_normal((2, 130, 16)).astype(np.float32)
    check_workload(ss, orc, w, h0=h0, num_segments=segs, euler=True, label=f"Euler, h0, A zeros, segments={segs}")


def test_euler_differs_from_zoh(ss):
    """The flag reaches the kernels: the two rules give visibly different outputs."""
    import torch
    w = W.make_scan_inputs(1, 64, 64, 16, "f32", seed=302)
    note("[case] Euler vs ZOH differ")
    from test_gpu_parity import run_gpu
    ye, _ = run_gpu(ss, w, euler=True)
    yz, _ = run_gpu(ss, w, euler=False)
    torch.cuda.synchronize()
    assert np.max(np.abs(ye - yz)) > 1e-3


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N,Bt", [(4, 3), (7, 3), (12, 3), (16, 3), (16, 8)])
def test_euler_step(ss, orc, dtype, N, Bt):
    import torch
    rng = np.random.default_rng(400 + N + Bt)
    Dm = 130
    note(f"[case] Euler step B={Bt} D={Dm} N={N} {dtype}")
    st0 = (0.3 * rng.standard_normal((Bt, Dm, N))).astype(np.float32)
    A = -(rng.uniform(0.5, 4, (Dm, N))).astype(np.float32)
    A[9, 1] = 0.0
    D = rng.standard_normal(Dm).astype(np.float32)
    bias = rng.uniform(-1, 1, Dm).astype(np.float32)
    st_gpu = f32dev(st0)
    st_ref = st0.astype(np.float64)
    tau = TAU[dtype]
    store = (lambda a: W.round_bf16(a)) if dtype == "bf16" else (lambda a: a.astype(np.float32))
    for k in range(5):
        x, dt, z = (store(rng.standard_normal((Bt, Dm))) for _ in range(3))
        Bm, Cm = (store(rng.standard_normal((Bt, N))) for _ in range(2))
        y = ss.sscan_step(st_gpu, tdev(x, dtype), tdev(dt, dtype), f32dev(A), tdev(Bm, dtype), tdev(Cm, dtype),
                          D=f32dev(D), z=tdev(z, dtype), delta_bias=f32dev(bias), euler=True)
        yr = orc.sscan_step(st_ref, x, dt, A, Bm, Cm, D=D, z=z, dt_bias=bias, euler=True)
        assert_close(host(y), yr, tau, f"y step {k}")
    torch.cuda.synchronize()
    assert_close(host(st_gpu), st_ref, tau, "state")
