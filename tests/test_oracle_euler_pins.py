"""Pins for the oracle's Euler variant (Bbar = Delta B, the first-order rule of the
page-3 report's code, section 4.2: deltaB = delta * B; Abar stays exp(Delta A)).

As for the zero-order hold, each test checks the oracle against something other
than itself: scipy.signal.lfilter, numpy's convolution of the LTI kernel, a
brute-force unrolled sum, and the second-order agreement of the two rules as the
step size goes to zero.
"""
import numpy as np
import pytest
import scipy.signal
import scipy.special

from test_oracle_pins import rand_case, softplus_lib


def test_euler_first_order_filter_lfilter(oracle_mod):
    """N = 1, one channel, LTI: h = lfilter([Delta b], [1, -exp(Delta a)], x)."""
    rng = np.random.default_rng(31)
    L = 150
    x = rng.standard_normal(L)
    a, b, cc, v = -0.9, 0.7, 1.6, -0.8
    y, hl = oracle_mod.sscan_fwd(x.reshape(1, L, 1), np.full((1, L, 1), v), np.array([[a]]),
                                 np.full((1, L, 1), b), np.full((1, L, 1), cc), euler=True)
    delta = softplus_lib(v)
    h = scipy.signal.lfilter([delta * b], [1.0, -np.exp(delta * a)], x)
    np.testing.assert_allclose(y.ravel(), cc * h, rtol=1e-11, atol=1e-13)
    assert hl[0, 0, 0] == pytest.approx(h[-1], rel=1e-11)


def test_euler_lti_convolution_kernel(oracle_mod):
    """Constant Delta, B, C: y_t - D x_t = sum_{l<=t} K_l x_{t-l} with
    K_l = sum_n C_n exp(Delta A_n)^l Delta B_n."""
    rng = np.random.default_rng(32)
    Bt, L, Dm, N = 2, 40, 3, 5
    c = rand_case(rng, Bt, L, Dm, N, with_z=False, lti=True)
    y, _ = oracle_mod.sscan_fwd(**c, euler=True)
    for b in range(Bt):
        for d in range(Dm):
            delta = softplus_lib(c["dt"][b, 0, d] + c["dt_bias"][d])
            K = np.zeros(L)
            for n in range(N):
                K += c["C"][b, 0, n] * np.exp(delta * c["A"][d, n]) ** np.arange(L) * delta * c["B"][b, 0, n]
            expect = np.convolve(K, c["x"][b, :, d])[:L] + c["D"][d] * c["x"][b, :, d]
            np.testing.assert_allclose(y[b, :, d], expect, rtol=1e-11, atol=1e-12)


def test_euler_ltv_unrolled_sum(oracle_mod):
    """Input-dependent Delta, B, C: h_t = sum_{j<=t} (prod_{s=j+1}^{t} Abar_s) Delta_j B_j x_j,
    y_t = (C_t h_t + D x_t) silu(z_t), by brute force."""
    rng = np.random.default_rng(33)
    Bt, L, Dm, N = 1, 18, 3, 4
    c = rand_case(rng, Bt, L, Dm, N)
    y, hl = oracle_mod.sscan_fwd(**c, euler=True)
    for d in range(Dm):
        delta = softplus_lib(c["dt"][0, :, d] + c["dt_bias"][d])
        abar = np.exp(delta[:, None] * c["A"][d][None, :])
        for t in range(L):
            h = np.zeros(N)
            for j in range(t + 1):
                h += np.prod(abar[j + 1:t + 1], axis=0) * delta[j] * c["B"][0, j] * c["x"][0, j, d]
            zt = c["z"][0, t, d]
            expect = (c["C"][0, t] @ h + c["D"][d] * c["x"][0, t, d]) * zt * scipy.special.expit(zt)
            assert y[0, t, d] == pytest.approx(expect, rel=1e-11, abs=1e-12)
            if t == L - 1:
                np.testing.assert_allclose(hl[0, d], h, rtol=1e-11, atol=1e-13)


def test_euler_and_zoh_agree_to_second_order(oracle_mod):
    """One step from a zero state: y_zoh - y_euler = C x B (expm1(Delta A)/A - Delta)
    = C x B A Delta^2 / 2 + O(Delta^3); the ratio to the leading term tends to 1."""
    a, b, cc, xv = -3.0, 1.2, 0.9, 1.7
    ratios = []
    for delta in (1e-1, 1e-2, 1e-3):
        v = np.log(np.expm1(delta))
        args = (np.full((1, 1, 1), xv), np.full((1, 1, 1), v), np.array([[a]]), np.full((1, 1, 1), b),
                np.full((1, 1, 1), cc))
        yz, _ = oracle_mod.sscan_fwd(*args)
        ye, _ = oracle_mod.sscan_fwd(*args, euler=True)
        d_used = softplus_lib(v)
        ratios.append((yz[0, 0, 0] - ye[0, 0, 0]) / (cc * xv * b * a * d_used ** 2 / 2))
    assert abs(ratios[-1] - 1.0) < 2e-3
    assert abs(ratios[0] - 1.0) > abs(ratios[1] - 1.0) > abs(ratios[2] - 1.0)


def test_euler_step_equals_forward(oracle_mod):
    rng = np.random.default_rng(34)
    c = rand_case(rng, 2, 13, 4, 5)
    h0 = rng.standard_normal((2, 4, 5))
    y, hl = oracle_mod.sscan_fwd(**c, h0=h0, euler=True)
    st = h0.copy()
    for t in range(13):
        yt = oracle_mod.sscan_step(st, c["x"][:, t], c["dt"][:, t], c["A"], c["B"][:, t], c["C"][:, t],
                                   D=c["D"], z=c["z"][:, t], dt_bias=c["dt_bias"], euler=True)
        np.testing.assert_array_equal(yt, y[:, t])
    np.testing.assert_array_equal(st, hl)
