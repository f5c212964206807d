"""GPU parity of the fused convolution prologue (page-3 report, MambaBlock.forward and
step: causal depthwise conv1d over time + SiLU before the scan, with a cache of the
last d_conv - 1 raw inputs) against the oracle: conv_silu_prologue then the scan, in
fp64.  Same tolerances as the forward scan; the convolution state (raw inputs) must
match exactly."""
import numpy as np
import pytest

import workloads as W
from test_gpu_parity import TAU, assert_close, f32dev, host, note, orc, ss, tdev  # noqa: F401

pytestmark = pytest.mark.gpu


def conv_params(dim, K, seed, batch=None, with_state=True):
    rng = np.random.default_rng(seed)
    w = (0.5 * rng.standard_normal((dim, K))).astype(np.float32)
    cb = (0.1 * rng.standard_normal(dim)).astype(np.float32)
    st = rng.standard_normal((batch, dim, K - 1)).astype(np.float32) if with_state else None
    return w, cb, st


def check_conv_fwd(ss, orc, w, K, seed, with_state=True, euler=False, inplace=False, label=""):
    import torch
    cw, cb, cs = conv_params(w.dim, K, seed, w.batch, with_state)
    note(f"[case] conv fwd {label or w.name}: B={w.batch} L={w.seqlen} D={w.dim} N={w.dstate} K={K} {w.dtype} "
         f"state={with_state} euler={euler} inplace={inplace}")
    y = torch.empty(w.x.shape, dtype=torch.float32 if w.dtype == "f32" else torch.bfloat16, device="cuda")
    st = torch.empty((w.batch, w.dim, w.dstate), dtype=torch.float32, device="cuda")
    cin = f32dev(cs)
    cout = cin if (inplace and cin is not None) else torch.full((w.batch, w.dim, K - 1), float("nan"), device="cuda")
    ss.sscan_fwd(tdev(w.x, w.dtype), tdev(w.dt, w.dtype), f32dev(w.A), tdev(w.B, w.dtype), tdev(w.C, w.dtype),
                 D=f32dev(w.D), z=tdev(w.z, w.dtype), delta_bias=f32dev(w.dt_bias), out=y, last_state=st,
                 euler=euler, conv_w=f32dev(cw), conv_b=f32dev(cb), conv_state_in=cin, conv_state_out=cout)
    torch.cuda.synchronize()
    u, cs_ref = orc.conv_silu_prologue(w.x, cw, cb, cs)
    yr, sr = orc.sscan_fwd(u, w.dt, w.A, w.B, w.C, D=w.D, z=w.z, dt_bias=w.dt_bias, euler=euler)
    tau = TAU[w.dtype]
    ey = assert_close(host(y), yr, tau, "y")
    es = assert_close(host(st), sr, tau, "last_state")
    np.testing.assert_array_equal(host(cout), cs_ref.astype(np.float32))
    note(f"       max rel err y={ey:.3e} state={es:.3e}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_conv_fwd_ragged(ss, orc, dtype, K):
    w = W.make_scan_inputs(2, 53, 100, 16, dtype, seed=700 + K, name=f"conv ragged K={K}")
    check_conv_fwd(ss, orc, w, K, seed=K)


@pytest.mark.parametrize("with_state", [False, True])
def test_conv_fwd_segments_and_small_n(ss, orc, with_state):
    # L 300 over few channel tiles: the scan is split into segments (aggregate pass
    # reads the convolution output too); N = 5 exercises phantom states
    w = W.make_scan_inputs(2, 300, 130, 5, "f32", seed=710, name="conv segments")
    check_conv_fwd(ss, orc, w, 4, seed=11, with_state=with_state)


def test_conv_fwd_euler(ss, orc):
    w = W.make_scan_inputs(1, 90, 64, 16, "bf16", seed=711, name="conv Euler")
    check_conv_fwd(ss, orc, w, 4, seed=12, euler=True)


@pytest.mark.parametrize("L", [1, 2, 3])
def test_conv_fwd_sequence_shorter_than_window(ss, orc, L):
    w = W.make_scan_inputs(2, L, 64, 16, "f32", seed=712 + L, name=f"conv L={L}")
    check_conv_fwd(ss, orc, w, 4, seed=13, inplace=True, label=f"L={L} in-place state")


@pytest.mark.timeout(600)
def test_conv_fwd_mamba130m_layer(ss, orc):
    check_conv_fwd(ss, orc, W.workload("mamba130m_layer"), 4, seed=14)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [12, 16])
def test_conv_prefill_then_decode(ss, orc, dtype, N):
    """Prefill k tokens with the fused forward, hand the scan state and the
    convolution cache to the decode step, step the rest: equals the oracle over the
    whole sequence (page-3 report, sections 3 and 6).  N = 12: the decode step's
    second lane of a row holds one group of 4 states and none past it."""
    import torch
    w = W.make_scan_inputs(2, 40, 96, N, dtype, seed=720, name="prefill + decode")
    K, k = 4, 29
    cw, cb, _ = conv_params(w.dim, K, 21, w.batch, with_state=False)
    note(f"[case] conv prefill {k} + decode {w.seqlen - k} {dtype} N={N}")
    sl = lambda a, lo, hi: None if a is None else np.ascontiguousarray(a[:, lo:hi])
    st = torch.empty((w.batch, w.dim, w.dstate), dtype=torch.float32, device="cuda")
    cst = torch.empty((w.batch, w.dim, K - 1), dtype=torch.float32, device="cuda")
    y1 = ss.sscan_fwd(tdev(sl(w.x, 0, k), dtype), tdev(sl(w.dt, 0, k), dtype), f32dev(w.A),
                      tdev(sl(w.B, 0, k), dtype), tdev(sl(w.C, 0, k), dtype), D=f32dev(w.D),
                      z=tdev(sl(w.z, 0, k), dtype), delta_bias=f32dev(w.dt_bias), last_state=st,
                      conv_w=f32dev(cw), conv_b=f32dev(cb), conv_state_out=cst)
    ys = [host(y1)]
    for t in range(k, w.seqlen):
        yt = ss.sscan_step(st, tdev(w.x[:, t], dtype), tdev(w.dt[:, t], dtype), f32dev(w.A), tdev(w.B[:, t], dtype),
                           tdev(w.C[:, t], dtype), D=f32dev(w.D), z=tdev(w.z[:, t], dtype),
                           delta_bias=f32dev(w.dt_bias), conv_w=f32dev(cw), conv_b=f32dev(cb), conv_state=cst)
        ys.append(host(yt)[:, None, :])
    torch.cuda.synchronize()
    u, cs_ref = orc.conv_silu_prologue(w.x, cw, cb)
    yr, sr = orc.sscan_fwd(u, w.dt, w.A, w.B, w.C, D=w.D, z=w.z, dt_bias=w.dt_bias)
    tau = TAU[dtype]
    assert_close(np.concatenate(ys, axis=1), yr, tau, "y over prefill + decode")
    assert_close(host(st), sr, tau, "final scan state")
    np.testing.assert_array_equal(host(cst), cs_ref.astype(np.float32))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [7, 16])
def test_conv_fwd_long_row_layout(ss, orc, dtype, N):
    # L = 1000 over 2 x 100 channels: the sequence split gives segments of 9 chunks, each
    # run through the row-layout kernel's steady loop, with convolution windows that
    # reach back into the previous segment
    w = W.make_scan_inputs(2, 1000, 100, N, dtype, seed=730 + N, name=f"conv long N={N}")
    check_conv_fwd(ss, orc, w, 4, seed=31 + N)


@pytest.mark.timeout(600)
def test_conv_fwd_train_shape(ss, orc):
    # one workgroup per CU, one segment: 256 chunks of the row-layout kernel
    check_conv_fwd(ss, orc, W.workload("train_shape"), 4, seed=15)
