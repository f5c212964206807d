"""GPU parity of the checkpointed training path: sscan_fwd_checkpointed saves the
state entering every 8 timesteps, sscan_bwd_checkpointed starts its reverse pass from
those states (both through the C ABI).

  * the saved checkpoints equal the oracle's state after 8j steps (the forward run
    on the sequence prefix), elementwise within tau (1 + |h|);
  * y and the final state equal plain sscan_fwd's;
  * every gradient meets the backward pass's tolerances against the oracle.
"""
import numpy as np
import pytest

import workloads as W
from test_gpu_bwd import ELEMENTWISE, NORMWISE, upstream
from test_gpu_parity import TAU, assert_close, f32dev, host, note, orc, ss, tdev  # noqa: F401

pytestmark = pytest.mark.gpu


def run_fwd_ck(ss, w, h0=None, euler=False):
    import torch
    ck = torch.full((ss.checkpoint_bytes(w.batch, w.seqlen, w.dim, w.dstate) // 4,), float("nan"),
                    dtype=torch.float32, device="cuda")
    y, st = ss.sscan_fwd(tdev(w.x, w.dtype), tdev(w.dt, w.dtype), f32dev(w.A), tdev(w.B, w.dtype),
                         tdev(w.C, w.dtype), D=f32dev(w.D), z=tdev(w.z, w.dtype), delta_bias=f32dev(w.dt_bias),
                         initial_state=f32dev(h0), return_last_state=True, euler=euler, checkpoints=ck)
    torch.cuda.synchronize()
    return ck, y, st


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [3, 16])
@pytest.mark.parametrize("euler", [False, True])
def test_checkpoints_are_the_states(ss, orc, dtype, N, euler):
    # L 53: six full 8-step blocks and a tail; dim 100: a ragged channel tile
    w = W.make_scan_inputs(2, 53, 100, N, dtype, seed=900 + N, name=f"checkpoints N={N}")
    h0 = np.random.default_rng(N).standard_normal((2, 100, N)).astype(np.float32)
    note(f"[case] checkpoints B=2 L=53 D=100 N={N} {dtype} euler={euler}")
    ck, _, _ = run_fwd_ck(ss, w, h0=h0, euler=euler)
    nblk = (w.seqlen + 7) // 8
    ck = host(ck).reshape(w.batch, nblk, N, w.dim)
    tau = TAU[dtype]
    for j in range(nblk):
        l = 8 * j
        if l == 0:
            ref = h0.astype(np.float64)
        else:
            _, ref = orc.sscan_fwd(w.x[:, :l], w.dt[:, :l], w.A, w.B[:, :l], w.C[:, :l], D=w.D, z=w.z[:, :l],
                                   dt_bias=w.dt_bias, h0=h0, euler=euler)
        assert_close(np.transpose(ck[:, j], (0, 2, 1)), ref, tau, f"checkpoint {j}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [(2, 53, 100, 16), (2, 300, 130, 16), (1, 2000, 64, 8)])
def test_fwd_checkpointed_outputs_match_fwd(ss, dtype, shape):
    # the last two shapes have few workgroups: the forward splits the sequence
    import torch
    w = W.make_scan_inputs(*shape, dtype, seed=910, name="fwd checkpointed")
    note(f"[case] fwd checkpointed vs fwd {shape} {dtype}")
    _, y_ck, st_ck = run_fwd_ck(ss, w)
    y, st = ss.sscan_fwd(tdev(w.x, w.dtype), tdev(w.dt, w.dtype), f32dev(w.A), tdev(w.B, w.dtype),
                         tdev(w.C, w.dtype), D=f32dev(w.D), z=tdev(w.z, w.dtype), delta_bias=f32dev(w.dt_bias),
                         return_last_state=True)
    torch.cuda.synchronize()
    assert np.array_equal(host(y_ck), host(y)), "y differs from sscan_fwd"
    assert np.array_equal(host(st_ck), host(st)), "last state differs from sscan_fwd"


def check_bwd_ck(ss, orc, w, h0=None, with_dlast=True, euler=False, label=""):
    import torch
    note(f"[case] bwd checkpointed {label or w.name}: B={w.batch} L={w.seqlen} D={w.dim} N={w.dstate} "
         f"{w.dtype} euler={euler} h0={h0 is not None} dlast={with_dlast}")
    dy, dl = upstream(w, 78, with_dlast)
    ck, _, _ = run_fwd_ck(ss, w, h0=h0, euler=euler)
    g = ss.sscan_bwd(tdev(w.x, w.dtype), tdev(w.dt, w.dtype), f32dev(w.A), tdev(w.B, w.dtype), tdev(w.C, w.dtype),
                     tdev(dy, w.dtype), D=f32dev(w.D), z=tdev(w.z, w.dtype), delta_bias=f32dev(w.dt_bias),
                     dlast_state=f32dev(dl), euler=euler, checkpoints=ck)
    torch.cuda.synchronize()
    ref = orc.sscan_bwd(w.x, w.dt, w.A, w.B, w.C, dy, D=w.D, z=w.z, dt_bias=w.dt_bias, h0=h0, dlast_state=dl,
                        euler=euler)
    tau = TAU[w.dtype]
    worst = {}
    for name, rname in ELEMENTWISE.items():
        if g.get(name) is not None:
            worst[name] = assert_close(host(g[name]), ref[rname], tau, name)
    for name, rname in NORMWISE.items():
        if g.get(name) is None:
            continue
        got, r = host(g[name]).astype(np.float64), ref[rname]
        e = float(np.max(np.abs(got - r)) / (1.0 + np.max(np.abs(r))))
        assert e <= tau and np.all(np.isfinite(got)), f"{name}: normwise error {e:.3e} > tau={tau}"
        worst[name] = e
    note("       " + " ".join(f"{k}={v:.2e}" for k, v in worst.items()))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [1, 4, 16])
def test_bwd_checkpointed_ragged(ss, orc, dtype, N):
    w = W.make_scan_inputs(2, 53, 100, N, dtype, seed=920 + N, name=f"bwd ck ragged N={N}")
    h0 = np.random.default_rng(N + 1).standard_normal((2, 100, N)).astype(np.float32)
    check_bwd_ck(ss, orc, w, h0=h0)


@pytest.mark.parametrize("euler", [False, True])
def test_bwd_checkpointed_segments(ss, orc, euler):
    # few workgroups: the forward splits the sequence, and so does the reverse pass
    w = W.make_scan_inputs(2, 300, 130, 16, "f32", seed=930, name="bwd ck segments")
    h0 = np.random.default_rng(5).standard_normal((2, 130, 16)).astype(np.float32)
    check_bwd_ck(ss, orc, w, h0=h0, euler=euler, label="segments")


def test_bwd_checkpointed_no_dlast_no_gate(ss, orc):
    w = W.make_scan_inputs(1, 70, 64, 16, "bf16", seed=940, with_z=False, with_D=False, with_bias=False,
                           name="bwd ck minimal")
    check_bwd_ck(ss, orc, w, with_dlast=False)


@pytest.mark.timeout(600)
def test_bwd_checkpointed_mamba130m_layer(ss, orc):
    # 48 workgroups: split sequence in both directions
    check_bwd_ck(ss, orc, W.workload("mamba130m_layer"))


@pytest.mark.timeout(900)
def test_bwd_checkpointed_train_shape(ss, orc):
    check_bwd_ck(ss, orc, W.workload("train_shape"))


def test_checkpoints_rejected_with_conv_or_segments(ss):
    import torch
    w = W.make_scan_inputs(1, 16, 64, 4, "f32", seed=950, name="ck validation")
    args = (tdev(w.x, "f32"), tdev(w.dt, "f32"), f32dev(w.A), tdev(w.B, "f32"), tdev(w.C, "f32"))
    ck = torch.empty(ss.checkpoint_bytes(1, 16, 64, 4) // 4, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="checkpoints"):
        ss.sscan_fwd(*args, conv_w=torch.ones(64, 4, device="cuda"), checkpoints=ck)
    with pytest.raises(ValueError, match="checkpoints"):
        ss.sscan_fwd(*args, num_segments=2, checkpoints=ck)
    with pytest.raises(ss.SelScanError):     # one float short of the checkpoint array
        ss.sscan_fwd(*args, checkpoints=ck[1:])
