"""Pins for the fp64 oracle: each test checks it against something other than itself.

The pages print no numeric worked example, so the pins are: a hand-derived example
with exact rational values, closed forms, library routines that compute the same
object by a different method (scipy's matrix exponential for the zero-order hold,
scipy.signal.lfilter for a first-order recurrence, numpy's convolution for the LTI
kernel), brute-force unrolled sums on tiny inputs, and invariants (linearity, time
shift, step/forward equivalence, limits of the step size).

Together they are chosen so that a plausible slip in the oracle fails at least one:
Euler instead of ZOH (Van Loan pin), a sign error on A (worked example, lfilter),
an off-by-one in which state y reads (convolution pin, L=1 form), B and C swapped
(unrolled sum with distinct B, C), a dropped D or gate term (gate/skip pin, worked
example), a missing bias or a different softplus (softplus pin).
"""
import json
import os

import numpy as np
import pytest
import scipy.linalg
import scipy.integrate
import scipy.signal
import scipy.special

HERE = os.path.dirname(os.path.abspath(__file__))


def softplus_lib(v):
    """Library softplus: log(e^0 + e^v)."""
    return np.logaddexp(0.0, v)


def zoh_van_loan(a, b, delta):
    """Abar, Bbar for scalar dynamics a, input gain b and step delta, from the matrix
    exponential of the augmented system [[a, b], [0, 0]] * delta (Van Loan), which
    equals [[e^{a delta}, int_0^delta e^{a tau} d tau * b], [0, 1]]."""
    m = scipy.linalg.expm(np.array([[a * delta, b * delta], [0.0, 0.0]]))
    return m[0, 0], m[0, 1]


def rand_case(rng, batch, L, dim, N, with_z=True, with_D=True, with_bias=True, lti=False):
    x = rng.standard_normal((batch, L, dim))
    if lti:
        dt = np.broadcast_to(rng.uniform(-3, 0, (1, 1, dim)), (batch, L, dim)).copy()
        B = np.broadcast_to(rng.standard_normal((batch, 1, N)), (batch, L, N)).copy()
        C = np.broadcast_to(rng.standard_normal((batch, 1, N)), (batch, L, N)).copy()
    else:
        dt = rng.uniform(-4, 1, (batch, L, dim))
        B = rng.standard_normal((batch, L, N))
        C = rng.standard_normal((batch, L, N))
    A = -rng.uniform(0.2, 4.0, (dim, N))
    z = rng.standard_normal((batch, L, dim)) if with_z else None
    D = rng.standard_normal(dim) if with_D else None
    bias = rng.uniform(-1, 1, dim) if with_bias else None
    return dict(x=x, dt=dt, A=A, B=B, C=C, D=D, z=z, dt_bias=bias)


def test_hand_worked_example(oracle_mod):
    with open(os.path.join(HERE, "golden", "hand_worked_example.json")) as f:
        ex = json.load(f)
    Bt, L, Dm, N = ex["batch"], ex["seqlen"], ex["dim"], ex["dstate"]
    y, h = oracle_mod.sscan_fwd(np.reshape(ex["x"], (Bt, L, Dm)), np.reshape(ex["dt"], (Bt, L, Dm)),
                                np.array(ex["A"]), np.reshape(ex["B"], (Bt, L, N)),
                                np.reshape(ex["C"], (Bt, L, N)), D=np.array(ex["D"]),
                                dt_bias=np.array(ex["dt_bias"]))
    np.testing.assert_allclose(y.ravel(), ex["y_expected"], rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(h.ravel(), ex["last_state_expected"], rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("a", [-1.0, -16.0, -0.3, -1e-6, -250.0, 0.7])
@pytest.mark.parametrize("delta", [1e-4, 0.05, 1.3])
def test_zoh_against_van_loan_and_quadrature(oracle_mod, a, delta):
    """Two steps of one channel, one state: x = [1, 0], C = 1, no D, no gate.
    y_0 = Bbar_0 and y_1 = Abar_1 * Bbar_0 expose both ZOH factors."""
    b = 0.8
    v = np.log(np.expm1(delta))          # dt so that softplus(dt) = delta
    x = np.array([1.0, 0.0]).reshape(1, 2, 1)
    dt = np.full((1, 2, 1), v)
    y, h = oracle_mod.sscan_fwd(x, dt, np.array([[a]]), np.full((1, 2, 1), b), np.ones((1, 2, 1)))
    d_used = softplus_lib(v)
    abar, bbar = zoh_van_loan(a, b, d_used)
    quad = scipy.integrate.quad(lambda t: np.exp(a * t), 0.0, d_used, epsabs=0, epsrel=1e-13)[0] * b
    assert y[0, 0, 0] == pytest.approx(bbar, rel=1e-11, abs=1e-300)
    assert y[0, 0, 0] == pytest.approx(quad, rel=1e-10)
    assert y[0, 1, 0] == pytest.approx(abar * bbar, rel=1e-11, abs=1e-300)
    assert h[0, 0, 0] == pytest.approx(abar * bbar, rel=1e-11, abs=1e-300)


def test_euler_would_fail_zoh_pin(oracle_mod):
    """Guard on the pin itself: the Euler form Bbar = Delta * B differs from the
    ZOH value by far more than the tolerance used above, at a moderate step."""
    a, b, delta = -2.0, 1.0, 0.5
    _, bbar = zoh_van_loan(a, b, delta)
    assert abs(delta * b - bbar) / abs(bbar) > 0.3


def test_lti_convolution_kernel(oracle_mod):
    """Constant Delta, B, C (LTI): y_t - D x_t = sum_{l=0}^{t} K_l x_{t-l},
    K_l = sum_n C_n Abar_n^l Bbar_n.  This is the convolution form of the
    fakeeyes2wo page ("离散 SSM 的卷积形式"), shifted by one step because here y_t
    reads the state that already includes x_t (velog.io "Discretization")."""
    rng = np.random.default_rng(11)
    Bt, L, Dm, N = 2, 48, 3, 4
    c = rand_case(rng, Bt, L, Dm, N, with_z=False, with_D=True, with_bias=True, lti=True)
    y, _ = oracle_mod.sscan_fwd(**c)
    for b in range(Bt):
        for d in range(Dm):
            delta = softplus_lib(c["dt"][b, 0, d] + c["dt_bias"][d])
            K = np.zeros(L)
            for n in range(N):
                abar, bbar = zoh_van_loan(c["A"][d, n], c["B"][b, 0, n], delta)
                K += c["C"][b, 0, n] * abar ** np.arange(L) * bbar
            conv = np.convolve(K, c["x"][b, :, d])[:L]
            expect = conv + c["D"][d] * c["x"][b, :, d]
            np.testing.assert_allclose(y[b, :, d], expect, rtol=1e-11, atol=1e-12)


def test_ltv_unrolled_sum(oracle_mod):
    """Input-dependent Delta, B, C (LTV): brute-force unrolled sum
    h_t = sum_{j<=t} (prod_{s=j+1}^{t} Abar_s) Bbar_j x_j (the fakeeyes2wo unrolled
    form with the per-step Abar_k, Bbar_k of its "引入可变步长" section), y_t = C_t h_t
    + D x_t, gated by silu(z_t); ZOH factors from the matrix exponential."""
    rng = np.random.default_rng(12)
    Bt, L, Dm, N = 1, 20, 3, 3
    c = rand_case(rng, Bt, L, Dm, N)
    y, hl = oracle_mod.sscan_fwd(**c)
    for d in range(Dm):
        delta = softplus_lib(c["dt"][0, :, d] + c["dt_bias"][d])
        abar = np.zeros((L, N))
        bbar = np.zeros((L, N))
        for t in range(L):
            for n in range(N):
                abar[t, n], bbar[t, n] = zoh_van_loan(c["A"][d, n], c["B"][0, t, n], delta[t])
        for t in range(L):
            h = np.zeros(N)
            for j in range(t + 1):
                h += np.prod(abar[j + 1:t + 1], axis=0) * bbar[j] * c["x"][0, j, d]
            zt = c["z"][0, t, d]
            expect = (c["C"][0, t] @ h + c["D"][d] * c["x"][0, t, d]) * zt * scipy.special.expit(zt)
            assert y[0, t, d] == pytest.approx(expect, rel=1e-11, abs=1e-12)
            if t == L - 1:
                np.testing.assert_allclose(hl[0, d], h, rtol=1e-11, atol=1e-13)


def test_first_order_filter_lfilter(oracle_mod):
    """N = 1, one channel, LTI: the state is the first-order IIR filter
    h = lfilter([Bbar], [1, -Abar], x)."""
    rng = np.random.default_rng(13)
    L = 200
    x = rng.standard_normal(L)
    a, b, cc, v = -0.7, 1.3, -0.4, -1.2
    y, hl = oracle_mod.sscan_fwd(x.reshape(1, L, 1), np.full((1, L, 1), v), np.array([[a]]),
                                 np.full((1, L, 1), b), np.full((1, L, 1), cc))
    abar, bbar = zoh_van_loan(a, b, softplus_lib(v))
    h = scipy.signal.lfilter([bbar], [1.0, -abar], x)
    np.testing.assert_allclose(y.ravel(), cc * h, rtol=1e-11, atol=1e-13)
    assert hl[0, 0, 0] == pytest.approx(h[-1], rel=1e-11)


def test_linearity_in_x(oracle_mod):
    """Zero initial state, z fixed: y is linear in x."""
    rng = np.random.default_rng(14)
    c = rand_case(rng, 2, 33, 5, 4)
    x2 = rng.standard_normal(c["x"].shape)
    al, be = 1.7, -0.6
    y1, h1 = oracle_mod.sscan_fwd(**c)
    y2, h2 = oracle_mod.sscan_fwd(**{**c, "x": x2})
    y3, h3 = oracle_mod.sscan_fwd(**{**c, "x": al * c["x"] + be * x2})
    np.testing.assert_allclose(y3, al * y1 + be * y2, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(h3, al * h1 + be * h2, rtol=1e-10, atol=1e-12)


def test_small_step_keeps_state_ignores_input(oracle_mod):
    """Delta -> 0 (velog.io section 3.5: a small step keeps the state and ignores the
    input): Abar -> 1, Bbar -> 0, so y = D x silu(z) and the state stays at h0."""
    rng = np.random.default_rng(15)
    c = rand_case(rng, 1, 16, 4, 3)
    c["dt"] = np.full_like(c["dt"], -60.0)
    c["dt_bias"] = None
    h0 = rng.standard_normal((1, 4, 3)) * 0.0
    y, hl = oracle_mod.sscan_fwd(**c, h0=h0)
    expect = c["D"][None, None, :] * c["x"] * c["z"] * scipy.special.expit(c["z"])
    np.testing.assert_allclose(y, expect, rtol=1e-12, atol=1e-20)
    assert np.max(np.abs(hl)) < 1e-20


def test_large_step_resets_state(oracle_mod):
    """Delta -> infinity (a large step resets the state and focuses on the current
    input): Abar -> 0 and Bbar -> -B/A, so the scan is memoryless:
    y_t = (sum_n C_tn B_tn / (-A_n) + D) x_t silu(z_t)."""
    rng = np.random.default_rng(16)
    c = rand_case(rng, 1, 12, 3, 4)
    c["dt"] = np.full_like(c["dt"], 60.0)
    c["dt_bias"] = None
    c["A"] = -np.abs(c["A"]) - 1.0
    y, hl = oracle_mod.sscan_fwd(**c)
    gain = np.einsum("bln,dn->bld", c["B"] * c["C"], -1.0 / c["A"])
    expect = (gain + c["D"][None, None, :]) * c["x"] * c["z"] * scipy.special.expit(c["z"])
    np.testing.assert_allclose(y, expect, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(hl[0], (c["B"][0, -1][None, :] / -c["A"]) * c["x"][0, -1][:, None], rtol=1e-12)


def test_time_shift_invariance_lti(oracle_mod):
    """LTI system (constant Delta, B, C): delaying x by s steps delays y by s steps
    (time invariance, fakeeyes2wo page "时不变性")."""
    rng = np.random.default_rng(17)
    c = rand_case(rng, 1, 40, 3, 4, with_z=False, lti=True)
    s = 7
    y, _ = oracle_mod.sscan_fwd(**c)
    xs = np.concatenate([np.zeros((1, s, 3)), c["x"][:, :-s]], axis=1)
    ys, _ = oracle_mod.sscan_fwd(**{**c, "x": xs})
    np.testing.assert_allclose(ys[:, s:], y[:, :-s], rtol=1e-12, atol=1e-14)
    assert np.all(ys[:, :s] == 0.0)


def test_step_equals_forward(oracle_mod):
    """L single-token steps on a carried state (page-3 report, section 6) equal
    one forward scan from the same initial state."""
    rng = np.random.default_rng(18)
    c = rand_case(rng, 2, 17, 5, 6)
    h0 = rng.standard_normal((2, 5, 6))
    y, hl = oracle_mod.sscan_fwd(**c, h0=h0)
    st = h0.copy()
    for t in range(17):
        yt = oracle_mod.sscan_step(st, c["x"][:, t], c["dt"][:, t], c["A"], c["B"][:, t], c["C"][:, t],
                                   D=c["D"], z=c["z"][:, t], dt_bias=c["dt_bias"])
        np.testing.assert_array_equal(yt, y[:, t])
    np.testing.assert_array_equal(st, hl)


def test_initial_state_split(oracle_mod):
    """Scanning [0, k) then [k, L) from the carried state equals one scan of [0, L):
    the carry semantics a segmented scan relies on."""
    rng = np.random.default_rng(19)
    c = rand_case(rng, 2, 50, 4, 5)
    y, hl = oracle_mod.sscan_fwd(**c)
    k = 23
    first = {key: (v[:, :k] if (isinstance(v, np.ndarray) and v.ndim == 3 and key != "A") else v)
             for key, v in c.items()}
    rest = {key: (v[:, k:] if (isinstance(v, np.ndarray) and v.ndim == 3 and key != "A") else v)
            for key, v in c.items()}
    y1, h1 = oracle_mod.sscan_fwd(**first)
    y2, h2 = oracle_mod.sscan_fwd(**rest, h0=h1)
    np.testing.assert_array_equal(np.concatenate([y1, y2], axis=1), y)
    np.testing.assert_array_equal(h2, hl)


@pytest.mark.parametrize("A_value", [0.0, -1e-12])
def test_softplus_and_bias(oracle_mod, A_value):
    """With A = 0 (the ZOH limit Bbar = Delta B) or A tiny, y_0 = C B Delta x reveals
    Delta; it must equal the library softplus of dt + bias."""
    rng = np.random.default_rng(20)
    dts = np.array([-30.0, -5.0, -0.3, 0.0, 0.4, 3.0, 25.0])
    bias = np.array([0.25])
    for v in dts:
        y, _ = oracle_mod.sscan_fwd(np.full((1, 1, 1), 2.0), np.full((1, 1, 1), v), np.array([[A_value]]),
                                    np.full((1, 1, 1), 1.5), np.full((1, 1, 1), 0.5), dt_bias=bias)
        delta = y[0, 0, 0] / (2.0 * 1.5 * 0.5)
        # for A != 0, Bbar / B = Delta (1 + Delta A / 2 + ...): allow that first-order term
        assert delta == pytest.approx(softplus_lib(v + bias[0]), rel=1e-11 + 30 * abs(A_value))


def test_gate_and_skip_terms(oracle_mod):
    """y(z) = y(no z) * z * sigmoid(z), and y(D) - y(no D) = D x."""
    rng = np.random.default_rng(21)
    c = rand_case(rng, 2, 19, 4, 3)
    y, _ = oracle_mod.sscan_fwd(**c)
    y_nz, _ = oracle_mod.sscan_fwd(**{**c, "z": None})
    y_nzd, _ = oracle_mod.sscan_fwd(**{**c, "z": None, "D": None})
    np.testing.assert_allclose(y, y_nz * c["z"] * scipy.special.expit(c["z"]), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(y_nz - y_nzd, c["D"][None, None, :] * c["x"], rtol=1e-10, atol=1e-13)


def test_zero_A_is_continuous_limit(oracle_mod):
    rng = np.random.default_rng(22)
    c = rand_case(rng, 1, 30, 2, 3)
    c0 = {**c, "A": np.zeros_like(c["A"])}
    c1 = {**c, "A": np.full_like(c["A"], -1e-13)}
    y0, h0 = oracle_mod.sscan_fwd(**c0)
    y1, h1 = oracle_mod.sscan_fwd(**c1)
    np.testing.assert_allclose(y0, y1, rtol=1e-9, atol=1e-12)
    # with A = 0 the state is a plain running sum of Delta B x
    delta = softplus_lib(c["dt"] + c["dt_bias"][None, None, :])
    hsum = np.einsum("ld,ln->dn", delta[0] * c["x"][0], c["B"][0])
    np.testing.assert_allclose(h0[0], hsum, rtol=1e-10, atol=1e-12)


def test_thread_count_does_not_change_bits(oracle_mod):
    rng = np.random.default_rng(23)
    c = rand_case(rng, 3, 64, 37, 5)
    ya, ha = oracle_mod.sscan_fwd(**c, nthreads=1)
    yb, hb = oracle_mod.sscan_fwd(**c, nthreads=7)
    np.testing.assert_array_equal(ya, yb)
    np.testing.assert_array_equal(ha, hb)


def test_empty_and_degenerate_shapes(oracle_mod):
    rng = np.random.default_rng(24)
    # L = 0: no outputs, last state = initial state (zeros)
    y, h = oracle_mod.sscan_fwd(np.zeros((2, 0, 3)), np.zeros((2, 0, 3)), -np.ones((3, 4)),
                                np.zeros((2, 0, 4)), np.zeros((2, 0, 4)))
    assert y.shape == (2, 0, 3) and np.all(h == 0.0)
    # batch = 0
    y, h = oracle_mod.sscan_fwd(np.zeros((0, 5, 3)), np.zeros((0, 5, 3)), -np.ones((3, 4)),
                                np.zeros((0, 5, 4)), np.zeros((0, 5, 4)))
    assert y.shape == (0, 5, 3)


def test_fp64_accuracy_against_mpmath(oracle_mod):
    """Precision check (not a structural pin): the fp64 oracle agrees with a
    50-digit evaluation of the same recurrence to ~1e-14 relative on a tiny case."""
    mpmath = pytest.importorskip("mpmath")
    mpmath.mp.dps = 50
    rng = np.random.default_rng(25)
    c = rand_case(rng, 1, 12, 2, 3)
    y, _ = oracle_mod.sscan_fwd(**c)
    for d in range(2):
        h = [mpmath.mpf(0)] * 3
        for t in range(12):
            v = mpmath.mpf(c["dt"][0, t, d]) + mpmath.mpf(c["dt_bias"][d])
            delta = mpmath.log(1 + mpmath.exp(v))
            acc = mpmath.mpf(0)
            for n in range(3):
                a = mpmath.mpf(c["A"][d, n])
                h[n] = mpmath.exp(delta * a) * h[n] + mpmath.expm1(delta * a) / a * mpmath.mpf(c["B"][0, t, n]) * mpmath.mpf(c["x"][0, t, d])
                acc += mpmath.mpf(c["C"][0, t, n]) * h[n]
            acc += mpmath.mpf(c["D"][d]) * mpmath.mpf(c["x"][0, t, d])
            zz = mpmath.mpf(c["z"][0, t, d])
            acc *= zz / (1 + mpmath.exp(-zz))
            assert y[0, t, d] == pytest.approx(float(acc), rel=1e-13, abs=1e-15)
