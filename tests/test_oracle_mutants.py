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
from oracle_bidir_pins import BIDIR_PINS
from oracle_bwd_pins import BWD_PINS
from oracle_sidecar_pins import SIDECAR_PINS
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


# Mistakes in the backward (anchors are searched from the function named
# first; the forward code is left as committed).
BWD_MUTANTS = {
    "bwd_drop_decay_term": ("ref_selective_scan_backward(",
                            "A[d * N + n] * a * h_prev[n]);", "0.0 * a * h_prev[n]);"),
    "bwd_no_sigmoid": ("ref_selective_scan_backward(",
                       "ddelta * ref_sigmoid(dt[t * D + d])", "ddelta"),
    "bwd_sigmoid_sign": ("static double ref_sigmoid",
                         "return 1.0 / (1.0 + exp(-v));", "return 1.0 / (1.0 + exp(v));"),
    "bwd_g_not_decayed": ("ref_selective_scan_backward(", "g[n] *= a;", "g[n] *= 1.0;"),
    "bwd_dA_uses_h_now": ("ref_selective_scan_backward(",
                          "+= g[n] * delta[i] * a * h_prev[n];", "+= g[n] * delta[i] * a * h_now[n];"),
    "bwd_dC_uses_h_prev": ("ref_selective_scan_backward(",
                           "+= dy * h_now[n];", "+= dy * h_prev[n];"),
    "bwd_dx_no_residual": ("ref_selective_scan_backward(", "(res_kind == 1 ? dv : 0.0)", "0.0"),
    "bwd_dy_ungated": ("ref_selective_scan_backward(",
                       "const double dy = res_kind ? s * dv : dv;", "const double dy = dv;"),
    "bwd_dB_without_delta": ("ref_selective_scan_backward(",
                             "+= g[n] * delta[i] * xv;", "+= g[n] * xv;"),
    "bwd_ds_uses_dy": ("ref_selective_scan_backward(", "pS[task] += dv * yv;",
                       "pS[task] += dy * yv;"),
    "bwd_dDskip_uses_dout": ("ref_selective_scan_backward(", "pD[b * D + d] += dy * xv;",
                             "pD[b * D + d] += dv * xv;"),
    "bwd_g_skips_readout": ("ref_selective_scan_backward(", "g[n] += dy * Cm[t * N + n];",
                            "g[n] += 0.0 * Cm[t * N + n];"),
    "bwd_ignores_dh_out": ("ref_selective_scan_backward(",
                           "g[n] = dh_out ? dh_out[(b * D + d) * N + n] : 0.0;", "g[n] = 0.0;"),
    "bwd_dx_without_delta": ("ref_selective_scan_backward(",
                             "dxv += g[n] * delta[i] * Bm[t * N + n];",
                             "dxv += g[n] * Bm[t * N + n];"),
    "bwd_same_direction": ("ref_selective_scan_backward(",
                           "for (int64_t i = len - 1; i >= 0; --i) {",
                           "for (int64_t i = 0; i < len; ++i) {"),
}


# Mistakes in the bidirectional combination (anchors searched from its name).
BIDIR_MUTANTS = {
    "bidir_drop_reverse": ("ref_bidir_scan(", "const double yv = yf[i] + yr[i];",
                           "const double yv = yf[i];"),
    "bidir_reverse_with_forward_params": ("ref_bidir_scan(", "x, dt_r, Bm_r, Cm_r, A_r, Dskip_r,",
                                          "x, dt_f, Bm_f, Cm_f, A_f, Dskip_f,"),
    "bidir_both_forward": ("ref_bidir_scan(", "rc = ref_selective_scan(1, batch",
                           "rc = ref_selective_scan(0, batch"),
    "bidir_reverse_from_h_in": ("ref_bidir_scan(", "delta_softplus, NULL, NULL, yr",
                                "delta_softplus, h_in, NULL, yr"),
    "bidir_no_h_out": ("ref_bidir_scan(", "delta_softplus, h_in, h_out, yf",
                       "delta_softplus, h_in, NULL, yf"),
    "bidir_ungated": ("ref_bidir_scan(", "out[i] = res[i] + s * yv;", "out[i] = res[i] + yv;"),
    "bidir_lost_gate_select": ("ref_bidir_scan(", "else if (s == 0.0)", "else if (0)"),
}


def _build_anchored(workdir, name, start, old, new):
    text = open(SRC).read()
    at = text.index(start)
    at = text.find(old, at)
    assert at >= 0, "mutation anchor not found: %s" % name
    src = os.path.join(workdir, name + ".c")
    with open(src, "w") as f:
        f.write(text[:at] + new + text[at + len(old):])
    so = os.path.join(workdir, name + ".so")
    oracle.build(src=src, out=so)
    return oracle.OracleLib(so)


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


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_some_backward_pin_catches_mutant(workdir, name):
    start, old, new = BWD_MUTANTS[name]
    text = open(SRC).read()
    at = text.index(start)
    assert text.find(old, at) >= 0, "mutation anchor not found: %s" % name
    at = text.find(old, at)
    src = os.path.join(workdir, name + ".c")
    with open(src, "w") as f:
        f.write(text[:at] + new + text[at + len(old):])
    so = os.path.join(workdir, name + ".so")
    oracle.build(src=src, out=so)
    lib = oracle.OracleLib(so)

    def bwd(*a, **k):
        return oracle.selective_scan_backward(*a, lib=lib, **k)

    for pin in BWD_PINS:   # the first failing pin is enough
        try:
            pin(bwd)
        except (AssertionError, ValueError, FloatingPointError):
            return
    pytest.fail("no backward pin catches the planted mistake %r" % name)


@pytest.mark.parametrize("name", sorted(BIDIR_MUTANTS))
def test_some_bidir_pin_catches_mutant(workdir, name):
    lib = _build_anchored(workdir, name, *BIDIR_MUTANTS[name])

    def bidir(*a, **k):
        return oracle.bidir_scan(*a, lib=lib, **k)

    for pin in BIDIR_PINS:
        try:
            pin(bidir)
        except (AssertionError, ValueError, FloatingPointError):
            return
    pytest.fail("no bidirectional pin catches the planted mistake %r" % name)


# Mistakes in the sidecar block (Python: a patched copy of oracle/__init__.py
# is executed as its own module, sharing the committed C build).
SIDECAR_MUTANTS = {
    "sidecar_taps_reversed": ("acc = acc + conv_w[:, K - 1 - j] * x[t + j]",
                              "acc = acc + conv_w[:, j] * x[t + j]"),
    "sidecar_conv_looks_left": ("""                if t + j < off[b + 1]:
                    acc = acc + conv_w[:, K - 1 - j] * x[t + j]""",
                                """                if t - j >= off[b]:
                    acc = acc + conv_w[:, K - 1 - j] * x[t - j]"""),
    "sidecar_no_conv_silu": ("u = _round_to(_silu(pre), store)", "u = _round_to(pre, store)"),
    "sidecar_gate_with_x": ("g = _round_to(y * _silu(z), store)", "g = _round_to(y * _silu(x), store)"),
    "sidecar_halves_swapped": ("x, z = xz[:, :di], xz[:, di:]", "z, x = xz[:, :di], xz[:, di:]"),
    "sidecar_no_dt_bias": ("_round_to(xdbl[:, :R] @ W_dt.T, store) + dt_bias[None, :]",
                           "_round_to(xdbl[:, :R] @ W_dt.T, store)"),
    "sidecar_B_C_swapped": ("Bm, Cm = xdbl[:, R:R + N], xdbl[:, R + N:R + 2 * N]",
                            "Cm, Bm = xdbl[:, R:R + N], xdbl[:, R + N:R + 2 * N]"),
    "sidecar_forward_scan": ("y = selective_scan(u, dt, Bm, Cm, A, Dskip, reverse=True,",
                             "y = selective_scan(u, dt, Bm, Cm, A, Dskip, reverse=False,"),
    "sidecar_ungated": ("hidden + s * o", "hidden + o"),
    "sidecar_conv_without_bias": ("acc = conv_b.copy()", "acc = 0.0 * conv_b"),
}


@pytest.mark.parametrize("name", sorted(SIDECAR_MUTANTS))
def test_some_sidecar_pin_catches_mutant(name):
    import types
    old, new = SIDECAR_MUTANTS[name]
    path = os.path.join(os.path.dirname(oracle.__file__), "__init__.py")
    text = open(path).read()
    assert text.count(old) == 1, "mutation anchor not found: %s" % name
    mod = types.ModuleType("oracle_mutant_" + name)
    mod.__file__ = path
    exec(compile(text.replace(old, new), path, "exec"), mod.__dict__)
    for pin in SIDECAR_PINS:
        try:
            pin(mod.sidecar_forward)
        except (AssertionError, ValueError, FloatingPointError):
            return
    pytest.fail("no sidecar pin catches the planted mistake %r" % name)
