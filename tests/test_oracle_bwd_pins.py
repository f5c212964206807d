"""Pins for the oracle's backward pass (gradients of a scalar loss through the scan).

Each test ties the backward oracle to something other than itself:
  * central finite differences of the (separately pinned) forward oracle, for
    every input, for both discretization rules, with and without the optional
    inputs, across the step-size regimes where dphi/dA switches formulation;
  * the adjoint (dot-product) identity of the map x -> (y, last state), which is
    linear when the gate is absent and the initial state is zero;
  * closed forms for a single step;
  * a 50-digit evaluation of dLoss/dA where Delta*A is tiny (the regime where a
    cancelling formula would lose digits).
"""
import numpy as np
import pytest
import scipy.special

from test_oracle_pins import softplus_lib


def make_case(rng, Bt, L, Dm, N, with_z=True, with_D=True, with_bias=True, with_h0=True, with_dhl=True):
    c = dict(x=rng.standard_normal((Bt, L, Dm)), dt=rng.uniform(-3.0, 1.0, (Bt, L, Dm)),
             A=-rng.uniform(0.2, 3.0, (Dm, N)), B=rng.standard_normal((Bt, L, N)),
             C=rng.standard_normal((Bt, L, N)),
             D=rng.standard_normal(Dm) if with_D else None,
             z=rng.standard_normal((Bt, L, Dm)) if with_z else None,
             dt_bias=rng.uniform(-1, 1, Dm) if with_bias else None,
             h0=rng.standard_normal((Bt, Dm, N)) if with_h0 else None)
    dy = rng.standard_normal((Bt, L, Dm))
    dhl = rng.standard_normal((Bt, Dm, N)) if with_dhl else None
    return c, dy, dhl


def loss(orc, c, dy, dhl, euler):
    y, hl = orc.sscan_fwd(c["x"], c["dt"], c["A"], c["B"], c["C"], D=c["D"], z=c["z"], dt_bias=c["dt_bias"],
                          h0=c["h0"], euler=euler)
    out = float(np.sum(dy * y))
    if dhl is not None:
        out += float(np.sum(dhl * hl))
    return out


def finite_difference(orc, c, dy, dhl, euler, key, eps=1e-6):
    base = c[key]
    g = np.zeros_like(base)
    it = np.nditer(base, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        up, dn = base.copy(), base.copy()
        up[i] += eps
        dn[i] -= eps
        g[i] = (loss(orc, {**c, key: up}, dy, dhl, euler) - loss(orc, {**c, key: dn}, dy, dhl, euler)) / (2 * eps)
    return g


GRAD_OF = {"x": "dx", "dt": "ddt", "A": "dA", "B": "dB", "C": "dC", "D": "dD", "z": "dz", "dt_bias": "ddt_bias",
           "h0": "dh0"}


def check_against_fd(orc, c, dy, dhl, euler, tol=2e-8):
    g = orc.sscan_bwd(c["x"], c["dt"], c["A"], c["B"], c["C"], dy, D=c["D"], z=c["z"], dt_bias=c["dt_bias"],
                      h0=c["h0"], dlast_state=dhl, euler=euler)
    for key, gname in GRAD_OF.items():
        if c.get(key) is None:
            continue
        fd = finite_difference(orc, c, dy, dhl, euler, key)
        scale = 1.0 + np.max(np.abs(fd))
        err = np.max(np.abs(fd - g[gname])) / scale
        assert err < tol, f"{gname}: finite-difference mismatch {err:.2e}"


@pytest.mark.parametrize("euler", [False, True])
def test_bwd_matches_finite_differences(oracle_mod, euler):
    rng = np.random.default_rng(41)
    c, dy, dhl = make_case(rng, 2, 6, 3, 4)
    check_against_fd(oracle_mod, c, dy, dhl, euler)


def test_bwd_finite_differences_optional_inputs_absent(oracle_mod):
    rng = np.random.default_rng(42)
    c, dy, dhl = make_case(rng, 1, 7, 2, 3, with_z=False, with_D=False, with_bias=False, with_h0=False,
                           with_dhl=False)
    check_against_fd(oracle_mod, c, dy, dhl, False)


@pytest.mark.parametrize("regime", ["tiny_u", "large_u", "zero_A"])
def test_bwd_finite_differences_step_regimes(oracle_mod, regime):
    """dphi/dA switches between a series and a closed form at |Delta A| = 0.5, and A = 0
    uses the limit: check every regime, including both sides of the switch."""
    rng = np.random.default_rng(43)
    c, dy, dhl = make_case(rng, 1, 6, 2, 4)
    if regime == "tiny_u":
        c["dt"] = rng.uniform(-9.0, -6.0, c["dt"].shape)      # Delta ~ 1e-4 .. 2.5e-3
        c["A"] = -np.array([[0.3, 1.0, 180.0, 230.0], [0.05, 0.5, 200.0, 400.0]])   # u on both sides of 0.5
    elif regime == "large_u":
        c["dt"] = rng.uniform(0.5, 2.0, c["dt"].shape)
        c["A"] = -rng.uniform(1.0, 6.0, c["A"].shape)
    else:
        c["A"][0, 1] = 0.0
        c["A"][1, :] = 0.0
    check_against_fd(oracle_mod, c, dy, dhl, False, tol=5e-8)


def test_bwd_adjoint_identity(oracle_mod):
    """Without the gate and from a zero state, x -> (y, last state) is linear, so for
    any dy, dhL: <dy, y(x)> + <dhL, h_L(x)> = <dx, x> exactly (up to rounding)."""
    rng = np.random.default_rng(44)
    c, dy, dhl = make_case(rng, 2, 30, 4, 5, with_z=False, with_h0=False)
    for euler in (False, True):
        y, hl = oracle_mod.sscan_fwd(c["x"], c["dt"], c["A"], c["B"], c["C"], D=c["D"], dt_bias=c["dt_bias"],
                                     euler=euler)
        g = oracle_mod.sscan_bwd(c["x"], c["dt"], c["A"], c["B"], c["C"], dy, D=c["D"], dt_bias=c["dt_bias"],
                                 dlast_state=dhl, euler=euler)
        lhs = np.sum(dy * y) + np.sum(dhl * hl)
        rhs = np.sum(g["dx"] * c["x"])
        assert lhs == pytest.approx(rhs, rel=1e-12, abs=1e-12)
        # the same identity for C: y is linear in C (from a zero state, without the skip term)
        c0 = {**c, "D": None}
        y0, _ = oracle_mod.sscan_fwd(c0["x"], c0["dt"], c0["A"], c0["B"], c0["C"], dt_bias=c0["dt_bias"],
                                     euler=euler)
        g0 = oracle_mod.sscan_bwd(c0["x"], c0["dt"], c0["A"], c0["B"], c0["C"], dy, dt_bias=c0["dt_bias"],
                                  euler=euler)
        assert np.sum(dy * y0) == pytest.approx(np.sum(g0["dC"] * c0["C"]), rel=1e-12, abs=1e-12)
        # and for B (the state, hence y, is linear in B from a zero state)
        assert np.sum(dy * y0) == pytest.approx(np.sum(g0["dB"] * c0["B"]), rel=1e-12, abs=1e-12)


def test_bwd_single_step_closed_form(oracle_mod):
    """L = 1 from a zero state: y = (sum_n C_n phi_n B_n + D) x silu(z) with
    phi_n = expm1(Delta A_n)/A_n; every gradient but dA/dDelta has a one-line form."""
    rng = np.random.default_rng(45)
    N = 5
    x, v, zz, Dk = 0.8, -0.7, 0.6, 1.3
    A = -rng.uniform(0.5, 3.0, (1, N))
    Bv, Cv = rng.standard_normal(N), rng.standard_normal(N)
    dyv = -1.1
    g = oracle_mod.sscan_bwd(np.full((1, 1, 1), x), np.full((1, 1, 1), v), A, Bv.reshape(1, 1, N),
                             Cv.reshape(1, 1, N), np.full((1, 1, 1), dyv), D=np.array([Dk]),
                             z=np.full((1, 1, 1), zz))
    delta = softplus_lib(v)
    phi = np.expm1(delta * A[0]) / A[0]
    sg = scipy.special.expit(zz)
    s = zz * sg
    yo = (np.dot(Cv * phi, Bv) + Dk) * x
    gyo = dyv * s
    np.testing.assert_allclose(g["dC"].ravel(), gyo * phi * Bv * x, rtol=1e-13)
    np.testing.assert_allclose(g["dB"].ravel(), gyo * Cv * phi * x, rtol=1e-13)
    assert g["dx"].item() == pytest.approx(gyo * (np.dot(Cv * phi, Bv) + Dk), rel=1e-13)
    assert g["dD"].item() == pytest.approx(gyo * x, rel=1e-13)
    assert g["dz"].item() == pytest.approx(dyv * yo * (sg + zz * sg * (1 - sg)), rel=1e-13)
    # dLoss/dDelta = gyo x sum_n C_n B_n exp(Delta A_n) (d phi / d Delta = e^{Delta A})
    gdelta = gyo * x * np.dot(Cv * Bv, np.exp(delta * A[0]))
    assert g["ddt"].item() == pytest.approx(gdelta * scipy.special.expit(v), rel=1e-12)
    np.testing.assert_allclose(g["dh0"].ravel(), np.exp(delta * A[0]) * gyo * Cv, rtol=1e-13)


def test_bwd_dA_at_tiny_step_against_mpmath(oracle_mod):
    """dLoss/dA with Delta A ~ -1e-7 (deep in the cancelling regime), against a
    50-digit derivative of the two-step forward recurrence."""
    mpmath = pytest.importorskip("mpmath")
    mpmath.mp.dps = 50
    x = np.array([0.7, -1.2]).reshape(1, 2, 1)
    dt = np.array([-16.0, -15.5]).reshape(1, 2, 1)      # Delta ~ 1e-7
    Bv = np.array([0.9, -0.4]).reshape(1, 2, 1)
    Cv = np.array([1.1, 0.6]).reshape(1, 2, 1)
    a0 = -1.3
    dy = np.array([0.5, -0.8]).reshape(1, 2, 1)
    g = oracle_mod.sscan_bwd(x, dt, np.array([[a0]]), Bv, Cv, dy)

    def f(a):
        h = mpmath.mpf(0)
        tot = mpmath.mpf(0)
        for t in range(2):
            delta = mpmath.log(1 + mpmath.exp(mpmath.mpf(dt[0, t, 0])))
            h = mpmath.exp(delta * a) * h + mpmath.expm1(delta * a) / a * mpmath.mpf(Bv[0, t, 0]) * mpmath.mpf(x[0, t, 0])
            tot += mpmath.mpf(dy[0, t, 0]) * mpmath.mpf(Cv[0, t, 0]) * h
        return tot

    ref = mpmath.diff(f, mpmath.mpf(a0))
    assert g["dA"].item() == pytest.approx(float(ref), rel=1e-9)
