"""The fp64 oracle against what the mathematics fixes (CPU only)."""
import numpy as np
import pytest

import oracle
from oracle_bidir_pins import BIDIR_PINS
from oracle_bwd_pins import BWD_PINS
from oracle_sidecar_pins import SIDECAR_PINS
from oracle_pins import PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(oracle.selective_scan)


@pytest.mark.parametrize("pin", BIDIR_PINS, ids=[p.__name__ for p in BIDIR_PINS])
def test_bidir_pin(pin):
    pin(oracle.bidir_scan)


@pytest.mark.parametrize("pin", SIDECAR_PINS, ids=[p.__name__ for p in SIDECAR_PINS])
def test_sidecar_pin(pin):
    pin(oracle.sidecar_forward)


@pytest.mark.parametrize("pin", BWD_PINS, ids=[p.__name__ for p in BWD_PINS])
def test_backward_pin(pin):
    pin(oracle.selective_scan_backward)


def test_backward_thread_count_does_not_change_results():
    r = np.random.default_rng(2)
    T, D, N = 200, 130, 16
    args = (r.standard_normal((T, D)), r.normal(-2, 0.5, (T, D)), r.standard_normal((T, N)),
            r.standard_normal((T, N)), -np.tile(np.arange(1.0, 17.0), (D, 1)),
            r.standard_normal(D))
    kw = dict(reverse=True, dout=r.standard_normal((T, D)), seq_offsets=[0, 120, 120, 200],
              res_kind="x", s=0.2)
    a = oracle.selective_scan_backward(*args, nthreads=1, **kw)
    b = oracle.selective_scan_backward(*args, nthreads=8, **kw)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_thread_count_does_not_change_results():
    r = np.random.default_rng(0)
    x, dt = r.standard_normal((300, 7)), r.normal(-2, 0.5, (300, 7))
    Bm, Cm = r.standard_normal((300, 16)), r.standard_normal((300, 16))
    A = -np.tile(np.arange(1.0, 17.0), (7, 1))
    a = oracle.r2l_scan(x, dt, Bm, Cm, A, batch=3, seqlen=100, nthreads=1)["y"]
    b = oracle.r2l_scan(x, dt, Bm, Cm, A, batch=3, seqlen=100, nthreads=8)["y"]
    assert np.array_equal(a, b)


def test_rejects_bad_offsets():
    r = np.random.default_rng(0)
    x = r.standard_normal((6, 2))
    with pytest.raises(ValueError):
        oracle.r2l_scan(x, x, r.standard_normal((6, 3)), r.standard_normal((6, 3)),
                        -np.ones((2, 3)), seq_offsets=[0, 4, 2, 6])


def test_wrappers_match_general_routine():
    r = np.random.default_rng(1)
    x, dt = r.standard_normal((40, 3)), r.normal(-1, 0.5, (40, 3))
    Bm = r.standard_normal((40, 4))
    A = -np.ones((3, 4)) * np.arange(1.0, 5.0)
    h = oracle.prefix_scan_state(x, dt, Bm, A, batch=2, seqlen=20)
    h2 = oracle.block_commit_state(oracle.prefix_scan_state(x[:10], dt[:10], Bm[:10], A,
                                                            batch=1, seqlen=10),
                                   x[10:20], dt[10:20], Bm[10:20], A, batch=1, seqlen=10)
    assert np.array_equal(h[0], h2[0])
