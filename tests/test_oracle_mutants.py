"""The pins must catch plausible mistakes: compile deliberately broken copies of the
oracle's C source on the CPU and check that each one fails at least one pin."""
import inspect
import os
import shutil
import tempfile

import numpy as np
import pytest

import oracle
import test_oracle_bwd_pins as bwd_pins
import test_oracle_euler_pins as euler_pins
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "sscan_oracle.c")

# (name, original text, replacement) -- each a mistake someone could make.
MUTANTS = [
    ("euler_bbar", "expm1(a) / an * Bm[r + n]", "delta * Bm[r + n]"),
    ("abar_sign", "const double abar = exp(a);", "const double abar = exp(-a);"),
    ("bbar_sign", "expm1(a) / an * Bm[r + n]", "-expm1(a) / an * Bm[r + n]"),
    ("readout_before_update", "h[n] = abar * h[n] + bbar * xv;\n      acc += Cm[r + n] * h[n];",
     "acc += Cm[r + n] * h[n];\n      h[n] = abar * h[n] + bbar * xv;"),
    ("B_C_swapped", "acc += Cm[r + n] * h[n];", "acc += Bm[r + n] * h[n];"),
    ("dropped_skip", "if (Dskip) acc += Dskip[d] * xv;", "if (Dskip) acc += 0.0;"),
    ("dropped_bias", "const double bd = bias ? bias[d] : 0.0;", "const double bd = 0.0;"),
    ("softplus_is_exp", "return log1p(exp(v));", "return exp(v);"),
    ("gate_sigmoid_only", "return z / (1.0 + exp(-z));", "return 1.0 / (1.0 + exp(-z));"),
    ("input_not_scaled_by_x", "h[n] = abar * h[n] + bbar * xv;", "h[n] = abar * h[n] + bbar;"),
    ("state_not_decayed", "h[n] = abar * h[n] + bbar * xv;", "h[n] = h[n] + bbar * xv;"),
    ("delta_is_raw_dt", "const double delta = softplus(dt[i] + bd);", "const double delta = dt[i] + bd;"),
    ("A_index_transposed_square", "const double an = A[d * N + n];", "const double an = A[(n % Dm) * N + (d % N)];"),
    ("last_state_stale", "h_last[(b * Dm + d) * N + n] = h[n];", "h_last[(b * Dm + d) * N + n] = 0.0;"),
    ("euler_flag_ignored", "(an != 0.0 && !euler)", "(an != 0.0)"),
    ("euler_flag_inverted", "(an != 0.0 && !euler)", "(an != 0.0 && euler)"),
    # backward pass
    ("bwd_gradient_not_decayed", "gh[n] = abar * g;", "gh[n] = g;"),
    ("bwd_dB_missing_x", "dBm[r + n] += g * phi * xv;", "dBm[r + n] += g * phi;"),
    ("bwd_dC_previous_state", "dCm[r + n] += gyo * hs[(l + 1) * N + n];", "dCm[r + n] += gyo * hs[l * N + n];"),
    ("bwd_ddt_no_sigmoid", "const double gdt = gdelta * sigmoid(v);", "const double gdt = gdelta;"),
    ("bwd_dA_missing_input_term", "+ dphi_dA * Bm[r + n] * xv);", ");"),
    ("bwd_dz_sign", "(1.0 + zz * (1.0 - sg))", "(1.0 - zz * (1.0 - sg))"),
    ("bwd_series_factorial", "fact *= (double)(k + 3);", "fact *= (double)(k + 2);"),
    ("bwd_dx_missing_skip", "double gx = Dskip ? gyo * Dskip[d] : 0.0;", "double gx = 0.0;"),
    ("bwd_ddelta_decay_term_sign", "gdelta += g * (an * abar * hprev", "gdelta += g * (-an * abar * hprev"),
]


def _pin_functions():
    out = []
    members = (inspect.getmembers(pins, inspect.isfunction) + inspect.getmembers(euler_pins, inspect.isfunction)
               + inspect.getmembers(bwd_pins, inspect.isfunction))
    for name, fn in members:
        if not name.startswith("test_"):
            continue
        params = list(inspect.signature(fn).parameters)
        if params[0] != "oracle_mod":
            continue
        marks = getattr(fn, "pytestmark", [])
        cases = [{}]
        for m in marks:
            if m.name == "parametrize":
                argnames = [a.strip() for a in m.args[0].split(",")] if isinstance(m.args[0], str) else m.args[0]
                new = []
                for c in cases:
                    for v in m.args[1]:
                        vals = v if len(argnames) > 1 else (v,)
                        new.append({**c, **dict(zip(argnames, vals))})
                cases = new
        for c in cases:
            out.append((name, fn, c))
    return out


@pytest.fixture(scope="module")
def workdir():
    d = tempfile.mkdtemp(prefix="oracle_mutants_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(mutant, workdir):
    name, old, new = mutant
    src = open(SRC).read()
    assert old in src, f"mutation site for {name} not found"
    path = os.path.join(workdir, f"{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new, 1))
    lib = oracle.compile_source(path, os.path.join(workdir, f"lib{name}.so"))
    bad = oracle.Oracle(lib)
    caught = []
    for pname, fn, kwargs in _pin_functions():
        if pname == "test_fp64_accuracy_against_mpmath":
            continue  # a precision check, not counted as a pin
        try:
            with np.errstate(all="ignore"):
                fn(bad, **kwargs)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pname)
    assert caught, f"no pin catches mutant {name}"
