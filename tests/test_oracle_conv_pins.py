"""Pins for the oracle's convolution prologue (page-3 report, section 3: depthwise
conv1d over time with kernel d_conv, padding d_conv - 1, output cropped to the first
L steps, then SiLU; section 6: the step's cache of the last d_conv - 1 raw inputs).

Each test checks it against something other than itself: torch's conv1d with the
report's exact arguments, numpy's convolve per channel, and the cache handoff
(prefill in two pieces, or token by token, equals one prefill).
"""
import numpy as np
import pytest
import torch

import oracle


def case(rng, Bt=2, L=23, Dm=5, K=4, with_bias=True):
    return (rng.standard_normal((Bt, L, Dm)), rng.standard_normal((Dm, K)),
            rng.standard_normal(Dm) if with_bias else None)


@pytest.mark.parametrize("K", [1, 2, 4, 7])
def test_conv_matches_torch_conv1d_as_the_report_calls_it(K):
    rng = np.random.default_rng(60 + K)
    x, w, cb = case(rng, K=K)
    u, _ = oracle.conv_silu_prologue(x, w, cb)
    Bt, L, Dm = x.shape
    conv = torch.nn.Conv1d(Dm, Dm, kernel_size=K, groups=Dm, padding=K - 1, bias=True).double()
    with torch.no_grad():
        conv.weight.copy_(torch.from_numpy(w).reshape(Dm, 1, K))
        conv.bias.copy_(torch.from_numpy(cb))
        ref = torch.nn.functional.silu(conv(torch.from_numpy(x).transpose(1, 2))[:, :, :L]).transpose(1, 2)
    np.testing.assert_allclose(u, ref.numpy(), rtol=1e-13, atol=1e-14)


def test_conv_matches_numpy_convolve_per_channel():
    rng = np.random.default_rng(61)
    x, w, _ = case(rng, with_bias=False)
    u, _ = oracle.conv_silu_prologue(x, w)
    Bt, L, Dm = x.shape
    for b in range(Bt):
        for d in range(Dm):
            c = np.convolve(x[b, :, d], w[d, ::-1])[:L]     # causal: taps reversed, oldest first
            np.testing.assert_allclose(u[b, :, d], c / (1 + np.exp(-c)), rtol=1e-13, atol=1e-14)


def test_conv_cache_handoff_prefill_in_pieces():
    rng = np.random.default_rng(62)
    x, w, cb = case(rng, L=30)
    u, st = oracle.conv_silu_prologue(x, w, cb)
    u1, s1 = oracle.conv_silu_prologue(x[:, :11], w, cb)
    u2, s2 = oracle.conv_silu_prologue(x[:, 11:], w, cb, conv_state=s1)
    np.testing.assert_array_equal(np.concatenate([u1, u2], axis=1), u)
    np.testing.assert_array_equal(s2, st)
    # the state is the last K-1 raw inputs, oldest first
    np.testing.assert_array_equal(st, np.transpose(x[:, -3:, :], (0, 2, 1)))


def test_conv_cache_token_by_token_as_the_report_steps():
    """Report section 6: conv1d(cat([inputs, x]))[:, :, d_conv - 1], then the cache
    drops its oldest entry and appends x."""
    rng = np.random.default_rng(63)
    x, w, cb = case(rng, L=9)
    u, st = oracle.conv_silu_prologue(x, w, cb)
    Bt, L, Dm = x.shape
    K = w.shape[1]
    cache = np.zeros((Bt, Dm, K - 1))
    conv = torch.nn.Conv1d(Dm, Dm, kernel_size=K, groups=Dm, padding=K - 1, bias=True).double()
    with torch.no_grad():
        conv.weight.copy_(torch.from_numpy(w).reshape(Dm, 1, K))
        conv.bias.copy_(torch.from_numpy(cb))
        for t in range(L):
            xt = torch.from_numpy(x[:, t, :]).unsqueeze(2)
            full = torch.cat([torch.from_numpy(cache), xt], dim=2)
            c = conv(full)[:, :, K - 1]
            np.testing.assert_allclose(torch.nn.functional.silu(c).numpy(), u[:, t], rtol=1e-13, atol=1e-14)
            cache = torch.cat([torch.from_numpy(cache)[:, :, 1:], xt], dim=2).numpy()
    np.testing.assert_array_equal(cache, st)


def test_conv_short_sequence_keeps_part_of_the_old_state():
    rng = np.random.default_rng(64)
    x, w, cb = case(rng, L=2, K=5)
    s0 = rng.standard_normal((2, 5, 4))
    _, st = oracle.conv_silu_prologue(x, w, cb, conv_state=s0)
    np.testing.assert_array_equal(st[:, :, :2], s0[:, :, 2:])
    np.testing.assert_array_equal(st[:, :, 2:], np.transpose(x, (0, 2, 1)))
