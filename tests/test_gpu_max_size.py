"""GPU parity at sizes past 32-bit indexing.  Every token tensor of these calls holds
more than 2^31 elements (4.6 GB in bf16), so an element index or byte offset kept in
32 bits anywhere in the forward or backward path would leave outputs wrong or
unwritten.  Inputs are drawn on the device (workloads.device_scan_inputs: the
recipe of the named workloads, with Delta ~ logU[1e-3, 1e-1]).

The oracle runs on sampled (batch row, channel) pairs, since every channel of the
scan is independent: y, the last state and the per-token gradients dx, ddelta, dz of
(b, d) depend only on that channel's inputs, and dA[d], dD[d], ddelta_bias[d] sum over
the batch rows and steps of channel d only.  The sample covers the first channel
tile, tile edges, the middle and the last, partial tile (dim = 8200 = 128 x 64 + 8).
Outputs are filled with NaN before each call, and the whole of every output must
come back finite.  dB and dC sum over all channels, so they are only checked for
being finite here; the full training-shape test compares them element by element.
Tolerances are those of the other parity tests (bf16 inputs: tau = 2e-2).
"""
import numpy as np
import pytest

import workloads as W
from test_gpu_bwd import ELEMENTWISE, NORMWISE
from test_gpu_parity import TAU, assert_close, host, note, orc, ss  # noqa: F401

pytestmark = pytest.mark.gpu

SHAPE = (17, 16384, 8200, 16)          # batch, seqlen, dim, dstate: 2,283,929,600 elements per token tensor
ROWS = [0, 9, 16]
CHANS = [0, 1, 63, 64, 2047, 4096, 8191, 8192, 8199]
SEED = 45


@pytest.fixture(scope="module")
def big(ss):
    import torch
    Bt, L, Dm, N = SHAPE
    assert Bt * L * Dm > 2 ** 31
    note(f"[case] max size: B={Bt} L={L} D={Dm} N={N} bf16, device-drawn inputs seed={SEED}")
    t = W.device_scan_inputs(Bt, L, Dm, N, SEED)
    torch.cuda.synchronize()
    yield t
    del t
    torch.cuda.empty_cache()


def sample(t, rows=None):
    """Host float32 copy of a [batch, seqlen, dim] tensor at the sampled channels."""
    import torch
    idx = torch.tensor(CHANS, device=t.device)
    s = t.index_select(2, idx)
    if rows is not None:
        s = s.index_select(0, torch.tensor(rows, device=t.device))
    return host(s)


def test_forward_past_32bit_indexing(ss, orc, big):
    import torch
    t = big
    Bt, L, Dm, N = SHAPE
    y = torch.full_like(t["x"], float("nan"))
    st = torch.full((Bt, Dm, N), float("nan"), dtype=torch.float32, device="cuda")
    ss.sscan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"], delta_bias=t["dt_bias"], out=y,
                 last_state=st)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all()), "y has unwritten or non-finite elements"
    assert bool(torch.isfinite(st).all()), "last_state has unwritten or non-finite elements"
    ci = np.array(CHANS)
    A, D, bias = host(t["A"])[ci], host(t["D"])[ci], host(t["dt_bias"])[ci]
    B, C = host(t["B"])[ROWS], host(t["C"])[ROWS]
    yr, sr = orc.sscan_fwd(sample(t["x"], ROWS), sample(t["dt"], ROWS), A, B, C, D=D, z=sample(t["z"], ROWS),
                           dt_bias=bias)
    tau = TAU["bf16"]
    ey = assert_close(sample(y, ROWS), yr, tau, "y (sampled channels)")
    es = assert_close(host(st)[ROWS][:, ci, :], sr, tau, "last_state (sampled channels)")
    note(f"       max rel err y={ey:.3e} state={es:.3e} (tau {tau})")


def test_backward_past_32bit_indexing(ss, orc, big):
    import torch
    t = big
    Bt, L, Dm, N = SHAPE
    names = {"dx": (Bt, L, Dm), "ddelta": (Bt, L, Dm), "dz": (Bt, L, Dm), "dB": (Bt, L, N), "dC": (Bt, L, N)}
    out = {k: torch.full(s, float("nan"), dtype=torch.bfloat16, device="cuda") for k, s in names.items()}
    for k, s in {"dA": (Dm, N), "dD": (Dm,), "ddelta_bias": (Dm,), "dinitial_state": (Bt, Dm, N)}.items():
        out[k] = torch.full(s, float("nan"), dtype=torch.float32, device="cuda")
    g = ss.sscan_bwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["dy"], D=t["D"], z=t["z"], delta_bias=t["dt_bias"],
                     dlast_state=t["dlast"], out=out)
    torch.cuda.synchronize()
    for k in out:
        assert bool(torch.isfinite(g[k]).all()), f"{k} has unwritten or non-finite elements"
    ci = np.array(CHANS)
    A, D, bias = host(t["A"])[ci], host(t["D"])[ci], host(t["dt_bias"])[ci]
    ref = orc.sscan_bwd(sample(t["x"]), sample(t["dt"]), A, host(t["B"]), host(t["C"]), sample(t["dy"]), D=D,
                        z=sample(t["z"]), dt_bias=bias, dlast_state=host(t["dlast"])[:, ci, :])
    tau = TAU["bf16"]
    worst = {}
    for name, rname in ELEMENTWISE.items():
        if name in ("dB", "dC"):
            continue
        got = host(g[name])[:, ci, :] if name == "dinitial_state" else sample(g[name])
        worst[name] = assert_close(got, ref[rname], tau, f"{name} (sampled channels)")
    for name, rname in NORMWISE.items():
        got, r = host(g[name])[ci].astype(np.float64), ref[rname]
        err = float(np.max(np.abs(got - r)) / (1.0 + np.max(np.abs(r))))
        assert err <= tau, f"{name} (sampled channels): normwise error {err:.3e} above tau={tau}"
        worst[name] = err
    note("       max err " + " ".join(f"{k}={v:.3e}" for k, v in worst.items()) + f" (tau {tau})")


STEP_SHAPE = (8192, 16400, 16)         # batch, dim, dstate: 2,149,580,800 state elements (8.6 GB)
STEP_ROWS = [0, 4097, 8191]
STEP_CHANS = [0, 1, 5119, 5120, 16383, 16399]


def test_decode_step_past_32bit_indexing(ss, orc):
    """One sscan_step on a state of more than 2^31 elements; sampled (row, channel)
    pairs against the oracle's step (each (b, d) of the step is independent)."""
    import torch
    Bt, Dm, N = STEP_SHAPE
    assert Bt * Dm * N > 2 ** 31
    note(f"[case] max size step: B={Bt} D={Dm} N={N} bf16 tokens, fp32 state, device-drawn seed={SEED}")
    t = W.device_step_inputs(Bt, Dm, N, SEED)
    ri, ci = torch.tensor(STEP_ROWS, device="cuda"), torch.tensor(STEP_CHANS, device="cuda")
    st0 = t["state"].index_select(0, ri).index_select(1, ci).double().cpu().numpy().copy()
    y = torch.full_like(t["x"], float("nan"))
    ss.sscan_step(t["state"], t["x"], t["dt"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"], out=y)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all()), "y has unwritten or non-finite elements"
    assert bool(torch.isfinite(t["state"]).all()), "state has non-finite elements"

    def pick(a):
        return host(a.index_select(0, ri).index_select(1, ci))

    yr = orc.sscan_step(st0, pick(t["x"]), pick(t["dt"]), host(t["A"])[STEP_CHANS], host(t["B"].index_select(0, ri)),
                        host(t["C"].index_select(0, ri)), D=host(t["D"])[STEP_CHANS], z=pick(t["z"]))
    tau = TAU["bf16"]
    ey = assert_close(pick(y), yr, tau, "y (sampled rows and channels)")
    es = assert_close(host(t["state"].index_select(0, ri).index_select(1, ci)), st0, tau,
                      "state (sampled rows and channels)")
    note(f"       max rel err y={ey:.3e} state={es:.3e} (tau {tau})")
    del t, y
    torch.cuda.empty_cache()
