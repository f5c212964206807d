"""Oracle for the selective state-space scan (fp64, CPU).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package.  The product path (``selective_state_space_45_amd``) never calls it
and fails loudly when its HIP library is missing.  The oracle shares no code,
header, table or helper with the GPU path.

The arithmetic lives in ``sscan_oracle.c`` (plain C, fp64, libm ``exp``,
``expm1``, ``log1p``; OpenMP only splits independent (batch, channel) rows).
This module compiles it with gcc and marshals numpy arrays to it.

What it computes, and the passages it follows (the reference pages):

* Delta = softplus(dt + bias): velog.io Mamba review, section 3.2 "Improving SSMs
  with Selection" (project, add parameter, softplus; Delta has shape (B, L, D)).
* Zero-order hold for diagonal A, elementwise: Abar = exp(Delta A),
  Bbar = (Delta A)^-1 (exp(Delta A) - I) Delta B: velog.io review, section
  "2 State Space Models", "Discretization"; integral form on the fakeeyes2wo
  "mamba 学习" page, section "MAMBA".
* h_k = Abar h_{k-1} + Bbar x_k, y_k = C h_k (+ D x_k), then y * silu(z):
  velog.io review "Discretization" item 3; page-3 report sections 3 and 4.2.
* Recurrent step on a carried (B, D, N) state: page-3 report section 6 (ssm_step).
* ``euler=True``: Bbar = Delta B, the first-order rule of the page-3 report's code
  (section 4.2, ``deltaB = delta * B``).
* ``conv_silu_prologue``: the short causal depthwise convolution over time and the
  SiLU that precede the scan in the page-3 report's MambaBlock (section 3,
  ``forward``: conv1d with kernel d_conv and padding d_conv - 1, cropped to the
  first L outputs, then silu), with the convolution cache of its ``step``
  (section 6: the last d_conv - 1 raw inputs, oldest first).
* ``sscan_bwd``: gradients of a scalar loss with respect to every input, by the
  chain rule through the definition above, run backwards in time (the reverse
  recurrence that the page-3 report's ``pscan_rev`` serves, section 4.1).

Parity status: every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_pins.py`` (closed forms, a hand-derived worked example,
library routines, brute force and invariants).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sscan_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle_sscan.so")


def compile_source(src_path: str, out_path: str, verbose: bool = False) -> str:
    """Compile a C oracle source with gcc (no fast-math, no contraction) into a shared library."""
    tmp = out_path + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
           "-ffp-contract=off", "-o", tmp, src_path, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, out_path)
    return out_path


def build(verbose: bool = False) -> str:
    """Compile ``sscan_oracle.c`` into ``liboracle_sscan.so``."""
    return compile_source(_SRC, _LIB_PATH, verbose)


def _f64(a, shape=None, name="array"):
    if a is None:
        return None
    arr = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    if shape is not None and arr.shape != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {arr.shape}")
    return arr


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class Oracle:
    """ctypes front end of one compiled oracle library."""

    def __init__(self, lib_path: str):
        lib = ctypes.CDLL(lib_path)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.oracle_sscan_fwd.argtypes = [I64, I64, I64, I64, ctypes.c_int] + [P] * 11 + [ctypes.c_int]
        lib.oracle_sscan_fwd.restype = ctypes.c_int
        lib.oracle_sscan_step.argtypes = [I64, I64, I64, ctypes.c_int] + [P] * 10 + [ctypes.c_int]
        lib.oracle_sscan_step.restype = ctypes.c_int
        lib.oracle_sscan_bwd.argtypes = [I64, I64, I64, I64, ctypes.c_int] + [P] * 20 + [ctypes.c_int]
        lib.oracle_sscan_bwd.restype = ctypes.c_int
        lib.oracle_nthreads_default.argtypes = []
        lib.oracle_nthreads_default.restype = ctypes.c_int
        self.lib = lib
        self.last_threads_used = 0

    def default_threads(self) -> int:
        return int(self.lib.oracle_nthreads_default())

    def sscan_fwd(self, x, dt, A, B, C, D=None, z=None, dt_bias=None, h0=None,
                  return_last_state: bool = True, nthreads: int = 0, euler: bool = False
                  ) -> Tuple[np.ndarray, Optional[np.ndarray]]:
        """fp64 forward scan (``euler``: Bbar = Delta B instead of the zero-order hold).

        x, dt, z: [batch, seqlen, dim]; A: [dim, dstate]; B, C: [batch, seqlen, dstate];
        D, dt_bias: [dim]; h0: optional initial state [batch, dim, dstate] (zeros if None).
        Returns (y [batch, seqlen, dim], last_state [batch, dim, dstate] or None).
        """
        x = _f64(x, name="x")
        if x.ndim != 3:
            raise ValueError("x must be [batch, seqlen, dim]")
        Bt, L, Dm = x.shape
        A = _f64(A, name="A")
        if A.ndim != 2 or A.shape[0] != Dm:
            raise ValueError("A must be [dim, dstate]")
        N = A.shape[1]
        dt = _f64(dt, (Bt, L, Dm), "dt")
        B = _f64(B, (Bt, L, N), "B")
        C = _f64(C, (Bt, L, N), "C")
        D = _f64(D, (Dm,), "D")
        z = _f64(z, (Bt, L, Dm), "z")
        dt_bias = _f64(dt_bias, (Dm,), "dt_bias")
        h0 = _f64(h0, (Bt, Dm, N), "h0")
        y = np.empty((Bt, L, Dm), dtype=np.float64)
        hl = np.empty((Bt, Dm, N), dtype=np.float64) if return_last_state else None
        used = self.lib.oracle_sscan_fwd(Bt, L, Dm, N, int(bool(euler)), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C),
                                         _ptr(D), _ptr(z), _ptr(dt_bias), _ptr(h0), _ptr(y), _ptr(hl),
                                         int(nthreads))
        if used < 0:
            raise ValueError("oracle_sscan_fwd rejected its arguments")
        self.last_threads_used = used
        return y, hl

    def sscan_step(self, state, x, dt, A, B, C, D=None, z=None, dt_bias=None, nthreads: int = 0,
                   euler: bool = False):
        """fp64 single-token step.  ``state`` [batch, dim, dstate] (float64, C-contiguous)
        is updated in place; x, dt, z: [batch, dim]; B, C: [batch, dstate].  Returns y [batch, dim]."""
        if not (isinstance(state, np.ndarray) and state.dtype == np.float64 and state.flags.c_contiguous):
            raise TypeError("state must be a C-contiguous float64 numpy array (updated in place)")
        Bt, Dm, N = state.shape
        x = _f64(x, (Bt, Dm), "x")
        dt = _f64(dt, (Bt, Dm), "dt")
        A = _f64(A, (Dm, N), "A")
        B = _f64(B, (Bt, N), "B")
        C = _f64(C, (Bt, N), "C")
        D = _f64(D, (Dm,), "D")
        z = _f64(z, (Bt, Dm), "z")
        dt_bias = _f64(dt_bias, (Dm,), "dt_bias")
        y = np.empty((Bt, Dm), dtype=np.float64)
        used = self.lib.oracle_sscan_step(Bt, Dm, N, int(bool(euler)), _ptr(state), _ptr(x), _ptr(dt), _ptr(A), _ptr(B),
                                          _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias), _ptr(y), int(nthreads))
        if used < 0:
            raise ValueError("oracle_sscan_step rejected its arguments")
        self.last_threads_used = used
        return y


    def sscan_bwd(self, x, dt, A, B, C, dy, D=None, z=None, dt_bias=None, h0=None, dlast_state=None,
                  euler: bool = False, nthreads: int = 0) -> dict:
        """fp64 backward pass.  Same inputs as ``sscan_fwd`` plus dy [batch, seqlen, dim]
        (dLoss/dy) and optionally dlast_state [batch, dim, dstate] (dLoss/d last state).
        Returns a dict of gradients: dx, ddt, dz (if z), dA, dB, dC, dD (if D),
        ddt_bias (always; the gradient at bias = 0 when absent), dh0."""
        x = _f64(x, name="x")
        if x.ndim != 3:
            raise ValueError("x must be [batch, seqlen, dim]")
        Bt, L, Dm = x.shape
        A = _f64(A, name="A")
        if A.ndim != 2 or A.shape[0] != Dm:
            raise ValueError("A must be [dim, dstate]")
        N = A.shape[1]
        dt = _f64(dt, (Bt, L, Dm), "dt")
        B = _f64(B, (Bt, L, N), "B")
        C = _f64(C, (Bt, L, N), "C")
        dy = _f64(dy, (Bt, L, Dm), "dy")
        D = _f64(D, (Dm,), "D")
        z = _f64(z, (Bt, L, Dm), "z")
        dt_bias = _f64(dt_bias, (Dm,), "dt_bias")
        h0 = _f64(h0, (Bt, Dm, N), "h0")
        dhl = _f64(dlast_state, (Bt, Dm, N), "dlast_state")
        out = {"dx": np.empty((Bt, L, Dm)), "ddt": np.empty((Bt, L, Dm)), "dA": np.empty((Dm, N)),
               "dB": np.empty((Bt, L, N)), "dC": np.empty((Bt, L, N)),
               "dD": np.empty(Dm) if D is not None else None,
               "dz": np.empty((Bt, L, Dm)) if z is not None else None,
               "ddt_bias": np.empty(Dm), "dh0": np.empty((Bt, Dm, N))}
        used = self.lib.oracle_sscan_bwd(Bt, L, Dm, N, int(bool(euler)), _ptr(x), _ptr(dt), _ptr(A), _ptr(B),
                                         _ptr(C), _ptr(D), _ptr(z), _ptr(dt_bias), _ptr(h0), _ptr(dy),
                                         _ptr(dhl), _ptr(out["dx"]), _ptr(out["ddt"]), _ptr(out["dA"]),
                                         _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]), _ptr(out["dz"]),
                                         _ptr(out["ddt_bias"]), _ptr(out["dh0"]), int(nthreads))
        if used < 0:
            raise ValueError("oracle_sscan_bwd rejected its arguments")
        self.last_threads_used = used
        return out


def conv_silu_prologue(x, w, conv_bias=None, conv_state=None):
    """fp64 causal depthwise convolution over time followed by SiLU.

    x: [batch, seqlen, dim] raw inputs; w: [dim, dconv] filter taps (w[:, dconv-1]
    multiplies the current input, w[:, 0] the oldest); conv_bias: [dim] or None;
    conv_state: [batch, dim, dconv-1] raw inputs before x (oldest first), zeros if
    None.  Returns (u [batch, seqlen, dim], new_state [batch, dim, dconv-1]):
        c[b,l,d] = sum_k w[d,k] * xx[b, l + k, d] + conv_bias[d]
    where xx is x preceded along time by conv_state, and u = c * sigmoid(c); the new
    state is the last dconv - 1 entries of xx.  (Page-3 report, sections 3 and 6.)
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    Bt, L, Dm = x.shape
    K = w.shape[1]
    if w.shape[0] != Dm or K < 1:
        raise ValueError("w must be [dim, dconv]")
    st = (np.zeros((Bt, Dm, K - 1)) if conv_state is None
          else np.asarray(conv_state, dtype=np.float64).reshape(Bt, Dm, K - 1))
    xx = np.concatenate([np.transpose(st, (0, 2, 1)), x], axis=1)      # [batch, K-1+L, dim]
    c = np.zeros((Bt, L, Dm))
    for k in range(K):
        c += w[None, None, :, k] * xx[:, k:k + L, :]
    if conv_bias is not None:
        c += np.asarray(conv_bias, dtype=np.float64)[None, None, :]
    u = c / (1.0 + np.exp(-c))
    new_state = np.transpose(xx[:, L:, :], (0, 2, 1)).copy() if K > 1 else np.zeros((Bt, Dm, 0))
    return u, new_state


_default: Optional[Oracle] = None


def _load() -> Oracle:
    global _default
    if _default is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _default = Oracle(_LIB_PATH)
    return _default


def default_threads() -> int:
    return _load().default_threads()


def sscan_fwd(*args, **kwargs):
    """fp64 forward scan (see ``Oracle.sscan_fwd``)."""
    return _load().sscan_fwd(*args, **kwargs)


def sscan_step(*args, **kwargs):
    """fp64 single-token step (see ``Oracle.sscan_step``)."""
    return _load().sscan_step(*args, **kwargs)


def sscan_bwd(*args, **kwargs):
    """fp64 backward pass (see ``Oracle.sscan_bwd``)."""
    return _load().sscan_bwd(*args, **kwargs)


def last_threads_used() -> int:
    return _load().last_threads_used
