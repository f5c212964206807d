"""sscan_fwd_noalloc (the entry point for callers that cannot allocate) against
sscan_fwd with a caller workspace, through the C ABI.

Two calls in a row on the same GPU, the second on a smaller input, each with a
sequence split (so the static scratch array carries the split's carries, end
states and step sums): y and last_state must equal sscan_fwd's bit for bit (same
kernels, same split), and the fp64 oracle within the parity tolerance.  A shape
whose split would need more than SSCAN_NOALLOC_SCRATCH_BYTES is rejected before
anything runs.
"""
import ctypes

import numpy as np
import pytest

import workloads as W
from test_gpu_parity import TAU, assert_close, f32dev, host, note, orc, ss, tdev  # noqa: F401

pytestmark = pytest.mark.gpu


def run_both(ss, w, h0):
    import torch
    x, dt, z, B, C = (tdev(a, w.dtype) for a in (w.x, w.dt, w.z, w.B, w.C))
    A, D, bias, h0d = f32dev(w.A), f32dev(w.D), f32dev(w.dt_bias), f32dev(h0)
    need = ss.fwd_workspace_size(w.batch, w.seqlen, w.dim, w.dstate, x.dtype)
    assert 0 < need <= (32 << 20), need          # the case runs split, within the static scratch
    y_ref = torch.full_like(x, float("nan"))
    st_ref = torch.full((w.batch, w.dim, w.dstate), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    ss.sscan_fwd(x, dt, A, B, C, D=D, z=z, delta_bias=bias, initial_state=h0d, out=y_ref, last_state=st_ref,
                 workspace=ws)
    y = torch.full_like(x, float("nan"))
    st = torch.full((w.batch, w.dim, w.dstate), float("nan"), dtype=torch.float32, device="cuda")
    ss.sscan_fwd_noalloc(x, dt, A, B, C, D=D, z=z, delta_bias=bias, initial_state=h0d, out=y, last_state=st)
    torch.cuda.synchronize()
    return host(y), host(st), host(y_ref), host(st_ref)


def test_noalloc_matches_fwd_two_calls(ss, orc):
    cases = [W.make_scan_inputs(2, 3000, 256, 16, "bf16", seed=901, name="noalloc first call"),
             W.make_scan_inputs(1, 1000, 100, 16, "f32", seed=902, name="noalloc second call (smaller)")]
    for k, w in enumerate(cases):
        h0 = np.random.default_rng(903 + k).standard_normal((w.batch, w.dim, w.dstate)).astype(np.float32)
        note(f"[case] {w.name}: B={w.batch} L={w.seqlen} D={w.dim} N={w.dstate} {w.dtype} "
             f"scratch={ss.fwd_workspace_size(w.batch, w.seqlen, w.dim, w.dstate)} B")
        y, st, y_ref, st_ref = run_both(ss, w, h0)
        np.testing.assert_array_equal(y, y_ref)
        np.testing.assert_array_equal(st, st_ref)
        yr, sr = orc.sscan_fwd(w.x, w.dt, w.A, w.B, w.C, D=w.D, z=w.z, dt_bias=w.dt_bias, h0=h0)
        ey = assert_close(y, yr, TAU[w.dtype], "y")
        es = assert_close(st, sr, TAU[w.dtype], "last_state")
        note(f"       equal to sscan_fwd bit for bit; oracle err y={ey:.2e} state={es:.2e}")


def test_noalloc_rejects_scratch_above_the_maximum(ss):
    lib = ss.library()
    # batch 6, dim 1536 (24 channel tiles), seqlen 65536: the split picks 32 segments, so
    # carries, end states and sums take 38.9 MB > 32 MiB
    need = ss.fwd_workspace_size(6, 65536, 1536, 16)
    assert need > (32 << 20), need
    P = ctypes.c_void_p
    rc = lib.sscan_fwd_noalloc(6, 65536, 1536, 16, 1, 0, P(0x100000), P(0x200000), P(0x300000), P(0x400000),
                               P(0x500000), None, None, None, None, P(0x600000), None, None)
    assert rc == 1
    assert b"SSCAN_NOALLOC_SCRATCH_BYTES" in lib.sscan_last_error()
