"""Seeded input generator: determinism, storage exactness, and the stated distributions."""
import numpy as np

import workloads as W


def test_deterministic_and_seed_sensitive():
    a = W.workload("tiny")
    b = W.workload("tiny")
    c = W.workload("tiny", seed=99)
    for k in ("x", "dt", "z", "B", "C", "D"):
        np.testing.assert_array_equal(getattr(a, k), getattr(b, k))
    assert not np.array_equal(a.x, c.x)


def test_chunking_independent_of_threads(monkeypatch):
    big = W.make_scan_inputs(1, 3000, 2048, 4, "bf16", seed=7)   # > one 4 Mi chunk
    monkeypatch.setattr(W, "_THREADS", 1)
    one = W.make_scan_inputs(1, 3000, 2048, 4, "bf16", seed=7)
    np.testing.assert_array_equal(big.x, one.x)
    np.testing.assert_array_equal(big.dt, one.dt)


def test_bf16_values_are_exact():
    w = W.make_scan_inputs(2, 100, 64, 16, "bf16", seed=3)
    for k in ("x", "dt", "z", "B", "C"):
        u = getattr(w, k).view(np.uint32)
        assert np.all((u & 0xFFFF) == 0), k


def test_round_bf16_ties_to_even():
    # 1 + 2^-8 is halfway between bf16 neighbours 1 and 1 + 2^-7: ties to even -> 1
    # 1 + 3 * 2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: ties to even -> 1 + 2^-6
    v = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -20, -2.5], dtype=np.float32)
    r = W.round_bf16(v)
    np.testing.assert_array_equal(r, np.array([1.0, 1 + 2.0 ** -6, 1 + 2.0 ** -7, -2.5], dtype=np.float32))


def test_logu_step_sizes_land_in_range():
    w = W.make_scan_inputs(2, 512, 256, 16, "f32", seed=5, step="logu", delta_range=(1e-3, 1e-1))
    delta = np.logaddexp(0.0, w.dt.astype(np.float64) + w.dt_bias[None, None, :])
    assert delta.min() > 0.9e-3 and delta.max() < 1.1e-1
    # log-uniform: the median sits near the geometric mean 1e-2
    assert 0.7e-2 < np.median(delta) < 1.4e-2
    assert np.all(w.A == -np.arange(1, 17, dtype=np.float32)[None, :])


def test_decode_tokens_are_reproducible():
    dw = W.DecodeWorkload(batch=4, dim=64, dstate=16)
    t0 = dw.token(0)
    t0b = W.DecodeWorkload(batch=4, dim=64, dstate=16).token(0)
    t1 = dw.token(1)
    np.testing.assert_array_equal(t0.x, t0b.x)
    assert not np.array_equal(t0.x, t1.x)
    assert abs(float(dw.state0.std()) - 0.1) < 0.02


def test_algorithmic_bytes_of_the_training_shape():
    # x, dt, z read + y written at 2 bytes each, B and C, A, D and bias, the fp32 final state
    assert W.fwd_algorithmic_bytes(8, 4096, 2048, 16, "bf16") == (
        8 * 4096 * 2048 * 8 + 2 * 8 * 4096 * 16 * 2 + 4 * 2048 * 16 + 8 * 2048 + 4 * 8 * 2048 * 16)
