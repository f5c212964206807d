"""GPU parity of the backward pass (sscan_bwd, through the C ABI) against the fp64
oracle's backward pass on the same seeded inputs and upstream gradients.

Tolerances (tau = 1e-4 for fp32 inputs, 2e-2 for bf16 inputs, as for the forward):
  * per-token gradients dx, ddt, dz, the per-(b, l) gradients dB, dC and the
    initial-state gradient: elementwise |g - g_ref| <= tau (1 + |g_ref|);
  * dA, dD, ddelta_bias, which are sums over batch x sequence (up to 2^15 terms
    of both signs in fp32 registers): normwise, max|g - g_ref| <= tau (1 + max|g_ref|).
"""
import numpy as np
import pytest

import workloads as W
from test_gpu_parity import TAU, f32dev, host, note, orc, ss, tdev  # noqa: F401

pytestmark = pytest.mark.gpu

ELEMENTWISE = {"dx": "dx", "ddelta": "ddt", "dz": "dz", "dB": "dB", "dC": "dC", "dinitial_state": "dh0"}
NORMWISE = {"dA": "dA", "dD": "dD", "ddelta_bias": "ddt_bias"}


def upstream(w, seed, with_dlast):
    rng = np.random.default_rng(seed)
    dy = rng.standard_normal((w.batch, w.seqlen, w.dim)).astype(np.float32)
    if w.dtype == "bf16":
        dy = W.round_bf16(dy)
    dl = rng.standard_normal((w.batch, w.dim, w.dstate)).astype(np.float32) if with_dlast else None
    return dy, dl


def check_bwd(ss, orc, w, h0=None, with_dlast=True, euler=False, label="", seed=77):
    import torch
    note(f"[case] bwd {label or w.name}: B={w.batch} L={w.seqlen} D={w.dim} N={w.dstate} {w.dtype} "
         f"euler={euler} h0={h0 is not None} dlast={with_dlast}")
    dy, dl = upstream(w, seed, with_dlast)
    g = ss.sscan_bwd(tdev(w.x, w.dtype), tdev(w.dt, w.dtype), f32dev(w.A), tdev(w.B, w.dtype), tdev(w.C, w.dtype),
                     tdev(dy, w.dtype), D=f32dev(w.D), z=tdev(w.z, w.dtype), delta_bias=f32dev(w.dt_bias),
                     initial_state=f32dev(h0), dlast_state=f32dev(dl), euler=euler)
    torch.cuda.synchronize()
    ref = orc.sscan_bwd(w.x, w.dt, w.A, w.B, w.C, dy, D=w.D, z=w.z, dt_bias=w.dt_bias, h0=h0, dlast_state=dl,
                        euler=euler)
    tau = TAU[w.dtype]
    worst = {}
    for name, rname in ELEMENTWISE.items():
        if g.get(name) is None:
            continue
        got, r = host(g[name]).astype(np.float64), ref[rname]
        assert got.shape == r.shape, (name, got.shape, r.shape)
        err = np.abs(got - r) / (1.0 + np.abs(r))
        bad = ~(err <= tau)
        if bad.any():
            i = np.unravel_index(int(np.argmax(np.where(np.isnan(err), np.inf, err))), err.shape)
            raise AssertionError(f"{name}: {int(bad.sum())}/{err.size} outside tau={tau}; worst at {i}: "
                                 f"gpu={got[i]!r} oracle={r[i]!r}")
        worst[name] = float(err.max()) if err.size else 0.0
    for name, rname in NORMWISE.items():
        if g.get(name) is None:
            continue
        got, r = host(g[name]).astype(np.float64), ref[rname]
        scale = 1.0 + (np.max(np.abs(r)) if r.size else 0.0)
        e = float(np.max(np.abs(got - r)) / scale) if r.size else 0.0
        assert e <= tau and np.all(np.isfinite(got)), f"{name}: normwise error {e:.3e} > tau={tau}"
        worst[name] = e
    note("       " + " ".join(f"{k}={v:.2e}" for k, v in worst.items()))
    return worst


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [1, 3, 4, 7, 8, 16])
def test_bwd_ragged(ss, orc, dtype, N):
    # dim 100: a full 64-channel tile and a ragged one; L 53: six 8-step blocks and a tail
    w = W.make_scan_inputs(2, 53, 100, N, dtype, seed=500 + N, name=f"bwd ragged N={N}")
    h0 = np.random.default_rng(N).standard_normal((2, 100, N)).astype(np.float32)
    check_bwd(ss, orc, w, h0=h0)


@pytest.mark.parametrize("euler", [False, True])
def test_bwd_segmented_checkpoints(ss, orc, euler):
    # few workgroups and L = 300: the checkpoint pass splits the sequence into segments
    w = W.make_scan_inputs(2, 300, 130, 16, "f32", seed=501, name="bwd segments")
    h0 = np.random.default_rng(9).standard_normal((2, 130, 16)).astype(np.float32)
    check_bwd(ss, orc, w, h0=h0, euler=euler)


# The checkpoint pass that also forms the reverse segment aggregates runs where the
# checkpoint sweep is one segment (at least one workgroup per CU: batch x 64-channel
# tiles in [256, 512) on 256 CUs) and the reverse pass has two segments of whole
# chunks.  (4, 90, 4096): 256 workgroups, reverse segments of 48 and 42 steps (the
# second ends in a ragged chunk).
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("euler", [False, True])
def test_bwd_aggregates_in_checkpoint_pass(ss, orc, dtype, euler):
    w = W.make_scan_inputs(4, 90, 4096, 16, dtype, seed=510, name="bwd checkpoint pass with aggregates")
    h0 = np.random.default_rng(10).standard_normal((4, 4096, 16)).astype(np.float32)
    check_bwd(ss, orc, w, h0=h0, euler=euler)


def test_bwd_aggregates_in_checkpoint_pass_small_A_no_gate(ss, orc):
    # the same path with no z (gy = dy) and no final-state gradient, and channels whose
    # waves take the small-|A| form of the step (A = 0 included)
    w = W.make_scan_inputs(4, 96, 4096, 16, "f32", seed=511, with_z=False, name="bwd checkpoint pass, small A")
    w.A = w.A.copy()
    w.A[8:12, :] = -1e-3
    w.A[300, 4] = 0.0
    w.A[2049, :] = -1e-5
    check_bwd(ss, orc, w, with_dlast=False)


# A split checkpoint pass whose segments the reverse pass shares (N = 16, fewer
# workgroups than CUs): every checkpoint workgroup also forms its segment's reverse
# aggregate and the separate aggregate sweep is skipped.  (2, 1000, 200): 8 workgroups
# per segment (a ragged channel tile), 13 segments of 80 steps for both passes, the
# last one 40 steps (a ragged chunk); an initial state, dLoss/d(last state), and
# channels whose waves take the small-|A| forms (A = 0 included).
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("euler", [False, True])
def test_bwd_shared_segments(ss, orc, dtype, euler):
    w = W.make_scan_inputs(2, 1000, 200, 16, dtype, seed=512, name="bwd shared segments")
    w.A = w.A.copy()
    w.A[64:68, :] = -1e-3
    w.A[130, 2] = 0.0
    h0 = np.random.default_rng(12).standard_normal((2, 200, 16)).astype(np.float32)
    check_bwd(ss, orc, w, h0=h0, euler=euler)


def test_bwd_shared_segments_no_gate(ss, orc):
    # the same path with no z (gy = dy) and no final-state gradient
    w = W.make_scan_inputs(2, 1000, 200, 16, "f32", seed=513, with_z=False, name="bwd shared segments, no gate")
    check_bwd(ss, orc, w, with_dlast=False)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_optional_inputs_absent(ss, orc, dtype):
    w = W.make_scan_inputs(1, 70, 64, 16, dtype, seed=502, with_z=False, with_D=False, with_bias=False,
                           name="bwd no z, D, bias, h0, dlast")
    check_bwd(ss, orc, w, with_dlast=False)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_zero_A(ss, orc, dtype):
    w = W.make_scan_inputs(2, 64, 128, 16, dtype, seed=503, name="bwd A with zeros")
    w.A = w.A.copy()
    w.A[5, 3] = 0.0
    w.A[70, :] = 0.0
    check_bwd(ss, orc, w)


def test_bwd_small_steps_series_regime(ss, orc):
    # Delta ~ 1e-4 .. 1e-2: |Delta A| crosses 0.5 only for the largest states
    w = W.make_scan_inputs(1, 96, 64, 16, "f32", seed=504, delta_range=(1e-4, 1e-2), name="bwd small steps")
    check_bwd(ss, orc, w)


def test_bwd_extreme_steps(ss, orc):
    w = W.make_scan_inputs(1, 48, 64, 16, "f32", seed=505, name="bwd extreme dt")
    dt = w.dt.copy()
    dt[:, :16] = -30.0
    dt[:, 16:32] = 30.0
    w.dt = dt
    w.dt_bias = None
    check_bwd(ss, orc, w)


def test_bwd_seqlen_one(ss, orc):
    check_bwd(ss, orc, W.make_scan_inputs(3, 1, 80, 16, "bf16", seed=506, name="bwd L=1"))


@pytest.mark.timeout(600)
def test_bwd_long_sequence_few_channels(ss, orc):
    # 2500 blocks in one workgroup row, segmented checkpoints over a long sequence
    w = W.make_scan_inputs(1, 20000, 64, 16, "f32", seed=507, delta_range=(1e-4, 1e-2), name="bwd long")
    check_bwd(ss, orc, w)


@pytest.mark.timeout(600)
def test_bwd_mamba130m_layer(ss, orc):
    check_bwd(ss, orc, W.workload("mamba130m_layer"))


@pytest.mark.timeout(900)
def test_bwd_train_shape(ss, orc):
    check_bwd(ss, orc, W.workload("train_shape"))


@pytest.mark.timeout(600)
def test_bwd_euler_mamba130m_layer(ss, orc):
    check_bwd(ss, orc, W.workload("mamba130m_layer"), euler=True)


def test_bwd_deterministic(ss):
    import torch
    w = W.make_scan_inputs(2, 200, 192, 16, "bf16", seed=508)
    note("[case] bwd determinism")
    dy, dl = upstream(w, 5, True)
    args = (tdev(w.x, "bf16"), tdev(w.dt, "bf16"), f32dev(w.A), tdev(w.B, "bf16"), tdev(w.C, "bf16"), tdev(dy, "bf16"))
    kw = dict(D=f32dev(w.D), z=tdev(w.z, "bf16"), delta_bias=f32dev(w.dt_bias), dlast_state=f32dev(dl))
    a = ss.sscan_bwd(*args, **kw)
    b = ss.sscan_bwd(*args, **kw)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k], b[k]), k


def test_bwd_seqlen_zero(ss):
    import torch
    note("[case] bwd L=0")
    x = torch.empty(2, 0, 64, device="cuda")
    BC = torch.empty(2, 0, 16, device="cuda")
    A = -torch.ones(64, 16, device="cuda")
    dl = torch.randn(2, 64, 16, device="cuda")
    g = ss.sscan_bwd(x, x, A, BC, BC, x, D=torch.ones(64, device="cuda"), dlast_state=dl)
    torch.cuda.synchronize()
    assert torch.count_nonzero(g["dA"]) == 0 and torch.count_nonzero(g["dD"]) == 0
    assert torch.equal(g["dinitial_state"], dl)


def test_bwd_rejects_missing_workspace(ss):
    import torch
    note("[case] bwd workspace too small")
    x = torch.zeros(1, 16, 64, device="cuda")
    BC = torch.zeros(1, 16, 16, device="cuda")
    with pytest.raises(ss.SelScanError) as ei:
        ss.sscan_bwd(x, x, -torch.ones(64, 16, device="cuda"), BC, BC, x,
                     workspace=torch.empty(256, dtype=torch.uint8, device="cuda"))
    assert ei.value.code == 1
