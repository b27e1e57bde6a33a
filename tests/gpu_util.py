"""Helpers of the GPU parity tests: device copies of seeded inputs and the
comparisons against the fp64 oracle.

Tolerances (the bar of the parity tests):
* fp32 inputs: max|err| / max|ref| <= 1e-5 on y, out and states.
* bf16 inputs (fp32 state): max|err| / max|y_ref| <= 2e-2 on y; and every
  bf16 output element within one bf16 ulp of the oracle's value plus the fp32
  bound 1e-5 * max|y_ref| (the kernel computes in fp32 and rounds once to
  bf16, so beyond the fp32 error it can only land on the other side of one
  rounding boundary); states (kept in fp32) max|err|/max|h| <= 1e-5.
* bit-exact classes: s == 0 outputs, index/flip (integer-exact inputs),
  resumed == full scans under one plan, repeated launches.
"""
from __future__ import annotations

import json
import os

import numpy as np
import pytest
import torch

TOL = {"f32": 1e-5, "bf16": 2e-2}
STATE_TOL = 1e-5
TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def dev(a, dtype="f32"):
    """numpy fp32 (holding exact values of the dtype) -> device tensor."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(TORCH_DTYPE[dtype]).to("cuda")


def dev32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")


def host(t) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = np.max(np.abs(ref)) if ref.size else 0.0
    if ref.size == 0:
        return 0.0
    return float(np.max(np.abs(got - ref)) / max(scale, 1e-30))


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |v| (8 significant bits)."""
    a = np.maximum(np.abs(np.asarray(v, dtype=np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def report(what, err, tol):
    """Append a measured parity error to $R2L_PARITY_REPORT (JSON lines), if set."""
    path = os.environ.get("R2L_PARITY_REPORT")
    if path:
        test = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
        with open(path, "a") as f:
            f.write(json.dumps({"test": test, "what": what, "err": err, "tol": tol}) + "\n")


def check_y(got_t, ref, dtype, what="y"):
    got = host(got_t).reshape(np.shape(ref))
    e = rel_err(got, ref)
    report(what, e, TOL[dtype])
    assert e <= TOL[dtype], "%s: max|err|/max|ref| = %.3e > %.1e" % (what, e, TOL[dtype])
    if dtype == "bf16" and np.size(ref):
        ref = np.asarray(ref, dtype=np.float64)
        slack = bf16_ulp(ref) + 1e-5 * np.max(np.abs(ref))
        worst = float(np.max(np.abs(got - ref) / slack))
        assert worst <= 1.0, "%s: an element is %.2f x (1 bf16 ulp + fp32 bound) off" % (what, worst)
    return e


def check_state(got_t, ref, what="state"):
    e = rel_err(host(got_t), ref)
    report(what, e, STATE_TOL)
    assert e <= STATE_TOL, "%s: max|err|/max|ref| = %.3e > %.1e" % (what, e, STATE_TOL)
    return e


def bits(t) -> np.ndarray:
    t = t.detach().to("cpu").contiguous()
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).numpy()


@pytest.fixture(scope="session")
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible MI355X; run them with -m 'not gpu' elsewhere")
    torch.zeros(1, device="cuda")
    return torch.device("cuda")
