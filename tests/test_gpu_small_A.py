"""GPU parity where the zero-order-hold factor phi = (exp(Delta A) - 1)/A is taken at a
small |Delta A| (velog.io Mamba review, "Discretization": Bbar = (Delta A)^-1
(exp(Delta A) - I) Delta B; fakeeyes2wo "mamba 学习", section "MAMBA", the ZOH
integral A^-1 (e^{A Delta} - I) B).

Channels with |A| in {1e-1, 1e-2, 1e-3, 1e-5} (and one A = 0) sit beside the
A = -(n + 1) channels.  In fp32 the difference exp(Delta A) - 1 keeps only
~ulp(1)/|Delta A| relative precision, and the k-form update h <- Abar (h + k) - k,
k = x B / A, adds a rounding error of order ulp(x B / A) per step; both grow without
bound as |A| -> 0 while h does not.  These cases pin the kernels' accurate branch
(zoh_phi: a Taylor polynomial of expm1(u)/u for small |u|) against the fp64
oracle, which forms expm1(Delta A)/A directly.  Each case runs long enough (2048
steps, Delta ~ logU[1e-3, 1e-1]) that a cancelling form would exceed the fp32
tolerance 1e-4 (an fp32 emulation of the k-form gave 3e-4 at A = -1e-2 and 0.3 at
A = -1e-5 on this step-size range).

Launch configurations covered: the row-layout forward (one segment), the
two-level split with the row-layout main pass (3 segments), the split whose main
pass runs fwd_kernel with two states per wave (more workgroups than CUs), the
checkpoint pass and the reverse kernel of sscan_bwd, the checkpointed pair, the
conv prologue, and the decode step.
"""
import numpy as np
import pytest

import workloads as W
from test_gpu_bwd import check_bwd
from test_gpu_parity import TAU, assert_close, check_workload, f32dev, host, note, orc, ss, tdev  # noqa: F401

pytestmark = pytest.mark.gpu

SMALL = (-1e-1, -1e-2, -1e-3, -1e-5)


def with_small_A(w, tile_stride=64):
    """A = -(n + 1) except: channel 0 of every 64-channel tile has all states at -1e-1,
    channel 1 at -1e-2, channel 2 at -1e-3, channel 3 at -1e-5, channel 4 cycles
    through all four over n, and channel 5 has A[., 0] = 0 (the limit phi = Delta)."""
    A = w.A.copy()
    for base in range(0, w.dim, tile_stride):
        for i, a in enumerate(SMALL):
            if base + i < w.dim:
                A[base + i, :] = a
        if base + 4 < w.dim:
            A[base + 4, :] = [SMALL[n % 4] for n in range(w.dstate)]
        if base + 5 < w.dim:
            A[base + 5, 0] = 0.0
    w.A = A.astype(np.float32)
    return w


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("segs", [1, 3])
def test_small_A_forward_row_layout(ss, orc, dtype, segs):
    # 2 x 2 channel tiles: the row-layout kernel runs unsplit (1 segment) and as the
    # main pass of the two-level split (3 segments; the aggregate pass runs fwd_kernel)
    w = with_small_A(W.make_scan_inputs(2, 2048, 128, 16, dtype, seed=601, name="small A"))
    check_workload(ss, orc, w, num_segments=segs, label=f"small A {dtype}, {segs} segment(s)")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_small_A_forward_two_states_per_wave(ss, orc, dtype):
    # 4 batch rows x 8 tiles x 9 segments = 288 workgroups > 256 CUs: the main pass runs
    # fwd_kernel with two states per wave (and a ragged last segment)
    w = with_small_A(W.make_scan_inputs(4, 1100, 512, 16, dtype, seed=602, name="small A split"))
    check_workload(ss, orc, w, num_segments=9, label=f"small A {dtype}, 9 segments")


@pytest.mark.parametrize("N", [5, 16])
def test_small_A_forward_initial_state_small_n(ss, orc, N):
    w = with_small_A(W.make_scan_inputs(1, 700, 100, N, "f32", seed=603 + N, name="small A, h0"))
    h0 = np.random.default_rng(5).standard_normal((1, 100, N)).astype(np.float32)
    check_workload(ss, orc, w, h0=h0, label=f"small A, initial state, N={N}")
    check_workload(ss, orc, w, h0=h0, num_segments=4, label=f"small A, initial state, N={N}, 4 segments")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_small_A_backward(ss, orc, dtype):
    # the checkpoint pass (row layout) and the reverse kernel take their accurate
    # branches; 2 tiles x 1 batch row gives a reverse split over several segments
    w = with_small_A(W.make_scan_inputs(1, 1024, 128, 16, dtype, seed=610, name="bwd small A"))
    check_bwd(ss, orc, w, label=f"small A {dtype}")


def test_small_A_backward_checkpointed(ss, orc):
    import torch
    w = with_small_A(W.make_scan_inputs(2, 512, 96, 16, "f32", seed=611, name="bwd small A, checkpoints"))
    note(f"[case] checkpointed fwd/bwd small A: B={w.batch} L={w.seqlen} D={w.dim}")
    x, dt, z, B, C = (tdev(a, "f32") for a in (w.x, w.dt, w.z, w.B, w.C))
    A, D, bias = f32dev(w.A), f32dev(w.D), f32dev(w.dt_bias)
    ck = torch.empty(ss.checkpoint_bytes(w.batch, w.seqlen, w.dim, w.dstate) // 4, dtype=torch.float32,
                     device="cuda")
    y = ss.sscan_fwd(x, dt, A, B, C, D=D, z=z, delta_bias=bias, checkpoints=ck)
    dy = np.random.default_rng(612).standard_normal(w.x.shape).astype(np.float32)
    g = ss.sscan_bwd(x, dt, A, B, C, f32dev(dy), D=D, z=z, delta_bias=bias, checkpoints=ck)
    torch.cuda.synchronize()
    yr, _ = orc.sscan_fwd(w.x, w.dt, w.A, w.B, w.C, D=w.D, z=w.z, dt_bias=w.dt_bias)
    assert_close(host(y), yr, TAU["f32"], "y")
    ref = orc.sscan_bwd(w.x, w.dt, w.A, w.B, w.C, dy, D=w.D, z=w.z, dt_bias=w.dt_bias)
    for name, rname in (("dx", "dx"), ("ddelta", "ddt"), ("dz", "dz"), ("dB", "dB"), ("dC", "dC")):
        assert_close(host(g[name]), ref[rname], TAU["f32"], name)
    for name, rname in (("dA", "dA"), ("dD", "dD"), ("ddelta_bias", "ddt_bias")):
        got, r = host(g[name]).astype(np.float64), ref[rname]
        e = float(np.max(np.abs(got - r)) / (1.0 + np.max(np.abs(r))))
        assert e <= TAU["f32"], f"{name}: normwise error {e:.3e}"


def test_small_A_conv_prologue(ss, orc):
    import torch
    w = with_small_A(W.make_scan_inputs(2, 1000, 128, 16, "f32", seed=613, name="conv small A"))
    K = 4
    rng = np.random.default_rng(614)
    cw = (0.5 * rng.standard_normal((w.dim, K))).astype(np.float32)
    cb = (0.1 * rng.standard_normal(w.dim)).astype(np.float32)
    note(f"[case] conv prologue small A: B={w.batch} L={w.seqlen} D={w.dim} K={K}")
    y, st = ss.sscan_fwd(tdev(w.x, "f32"), tdev(w.dt, "f32"), f32dev(w.A), tdev(w.B, "f32"), tdev(w.C, "f32"),
                         D=f32dev(w.D), z=tdev(w.z, "f32"), delta_bias=f32dev(w.dt_bias), return_last_state=True,
                         conv_w=f32dev(cw), conv_b=f32dev(cb))
    torch.cuda.synchronize()
    u, _ = orc.conv_silu_prologue(w.x, cw, cb)
    yr, sr = orc.sscan_fwd(u, w.dt, w.A, w.B, w.C, D=w.D, z=w.z, dt_bias=w.dt_bias)
    assert_close(host(y), yr, TAU["f32"], "y")
    assert_close(host(st), sr, TAU["f32"], "last_state")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("Bt", [2, 4])
def test_small_A_decode_steps(ss, orc, dtype, Bt):
    # batch 4: the N = 16 kernel that walks 4 batch rows per thread
    import torch
    rng = np.random.default_rng(620 + Bt)
    Dm, N, steps = 72, 16, 300
    A = -(np.arange(1, N + 1, dtype=np.float32))[None, :].repeat(Dm, 0)
    for i, a in enumerate(SMALL):
        A[i, :] = a
    A[4, :] = [SMALL[n % 4] for n in range(N)]
    A[5, 0] = 0.0
    D = rng.standard_normal(Dm).astype(np.float32)
    # Delta ~ 1e-3 .. 1e-1 through the bias (softplus^-1 of the target step size)
    target = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), Dm))
    bias = np.log(np.expm1(target)).astype(np.float32)
    store = (lambda a: W.round_bf16(a)) if dtype == "bf16" else (lambda a: a.astype(np.float32))
    st0 = np.zeros((Bt, Dm, N), np.float32)
    st_gpu, st_ref = f32dev(st0), st0.astype(np.float64)
    tau = TAU[dtype]
    note(f"[case] decode small A {dtype}: B={Bt} D={Dm} N={N} steps={steps}")
    worst = 0.0
    for k in range(steps):
        x, z = store(rng.standard_normal((Bt, Dm))), store(rng.standard_normal((Bt, Dm)))
        dt = store(0.3 * rng.standard_normal((Bt, Dm)))
        Bm, Cm = store(rng.standard_normal((Bt, N))), store(rng.standard_normal((Bt, N)))
        y = ss.sscan_step(st_gpu, tdev(x, dtype), tdev(dt, dtype), f32dev(A), tdev(Bm, dtype), tdev(Cm, dtype),
                          D=f32dev(D), z=tdev(z, dtype), delta_bias=f32dev(bias))
        yr = orc.sscan_step(st_ref, x, dt, A, Bm, Cm, D=D, z=z, dt_bias=bias)
        worst = max(worst, assert_close(host(y), yr, tau, f"y at step {k + 1}"))
    torch.cuda.synchronize()
    e = assert_close(host(st_gpu), st_ref, tau, "state")
    note(f"       max rel err y={worst:.3e} state={e:.3e}")
