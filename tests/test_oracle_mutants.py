"""Each planted mistake in the oracle's source must make at least one pin fail.

The mistakes are the plausible ones: a dropped term, a wrong sign, a wrong or
shifted index, a transposed operand, a swapped operand, a lost initial state,
a lost gate select. Every mutant is a copy of the committed C source with one
textual substitution, built with gcc into a temporary directory (CPU only).
"""
import os
import tempfile

import pytest

import oracle
from oracle_pins import PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "selective_scan_ref.c")

MUTANTS = {
    "drop_dskip": ("(Dskip ? Dskip[d] : 0.0) * xv", "0.0 * xv"),
    "swap_direction": ("reverse ? start + len - 1 - i : start + i",
                       "reverse ? start + i : start + len - 1 - i"),
    "softplus_sign": ("log1p(exp(-fabs(v)))", "log1p(exp(fabs(v)))"),
    "softplus_dropped_max": ("return pos + log1p", "return log1p"),
    "transpose_A": ("exp(delta * A[d * N + n])", "exp(delta * A[(n * D + d) % (D * N)])"),
    "decay_without_delta": ("exp(delta * A[d * N + n])", "exp(A[d * N + n])"),
    "input_without_delta": ("(delta * Bm[t * N + n]) * xv", "Bm[t * N + n] * xv"),
    "readout_uses_B": ("acc += Cm[t * N + n] * h[n]", "acc += Bm[t * N + n] * h[n]"),
    "state_index_shift": ("acc += Cm[t * N + n] * h[n]", "acc += Cm[t * N + n] * h[(n + 1) % N]"),
    "ignore_h_in": ("h_in ? h_in[(b * D + d) * N + n] : 0.0", "0.0"),
    "lost_gate_select": ("else if (s == 0.0)", "else if (0)"),
    "ungated_residual": ("res[t * D + d] + s * yv", "res[t * D + d] + yv"),
    "shifted_delta_token": ("const double raw = dt[t * D + d];",
                            "const double raw = dt[(t > start ? t - 1 : t) * D + d];"),
    "shifted_B_token": ("(delta * Bm[t * N + n]) * xv",
                        "(delta * Bm[(t > start ? t - 1 : t) * N + n]) * xv"),
    "sign_of_decay": ("exp(delta * A[d * N + n])", "exp(-delta * A[d * N + n])"),
    "state_never_updated": (
        "h[n] = abar * h[n] + (delta * Bm[t * N + n]) * xv;\n            }",
        "h[n] = h[n];\n            }\n            double hn_tmp = 0;"),
}


@pytest.fixture(scope="module")
def workdir():
    with tempfile.TemporaryDirectory() as d:
        yield d


def _build_mutant(workdir, name, old, new):
    text = open(SRC).read()
    assert text.count(old) >= 1, "mutation anchor not found: %s" % name
    mutated = text.replace(old, new, 1)
    src = os.path.join(workdir, name + ".c")
    with open(src, "w") as f:
        f.write(mutated)
    so = os.path.join(workdir, name + ".so")
    oracle.build(src=src, out=so)
    return oracle.OracleLib(so)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_some_pin_catches_mutant(workdir, name):
    old, new = MUTANTS[name]
    lib = _build_mutant(workdir, name, old, new)

    def scan(*a, **k):
        return oracle.selective_scan(*a, lib=lib, **k)

    caught = []
    for pin in PINS:
        try:
            pin(scan)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, "no pin catches the planted mistake %r" % name
