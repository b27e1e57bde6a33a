"""Pins of the oracle's bidirectional full-window scan (``oracle.bidir_scan``).

Each ``pin_*`` takes ``bidir``, a callable with the signature of
``oracle.bidir_scan``, and raises ``AssertionError`` when it disagrees with
what the mathematics fixes. The operation (a reading: the block-diffusion page
names full-window bidirectional Mamba scans without writing them out) is the
forward scan of x with one parameter set plus the reverse scan of the same x
with another, readouts added, then the gated residual.

* direction sums   -- A = 0, Delta = 1, one unit state: y_t is a prefix sum plus
                      twice a suffix sum (np.cumsum; exact), and h_out is the
                      forward total, not the reverse one
* unrolled form    -- the O(L^2 N) semiseparable sums of both directions, with
                      separate parameters and an initial state entering only the
                      forward direction (random inputs, ragged batch)
* flip             -- swapping the parameter sets and flipping time mirrors the
                      output (bit for bit: the two readouts add in either order)
* gate             -- s = 0 returns the residual bit for bit; s != 0 gives
                      res + s*y; no residual gives y
"""
from __future__ import annotations

import numpy as np

from oracle_pins import _rand, _rel, _unrolled, _unit_sum_inputs


def pin_bidir_direction_sums(bidir):
    for lengths in ([9], [5, 0, 1, 7, 3]):
        off = np.concatenate([[0], np.cumsum(lengths)])
        x, dt, Bm, Cm, A = _unit_sum_inputs(lengths, 4, 3, len(lengths))
        rev = {"Bm": 2.0 * Bm}                 # the reverse direction counts twice
        r = bidir(x, dt, Bm, Cm, A, None, rev=rev, seq_offsets=off, delta_softplus=False,
                  want_h_out=True)
        for b in range(len(lengths)):
            seg = slice(off[b], off[b + 1])
            xs = x[seg]
            expect = np.cumsum(xs, axis=0) + 2.0 * np.cumsum(xs[::-1], axis=0)[::-1]
            assert np.array_equal(r["y"][seg], expect)
            assert np.array_equal(r["out"][seg], expect)
            assert np.array_equal(r["h_out"][b, :, 0], xs.sum(axis=0))
            assert not np.any(r["h_out"][b, :, 1:])


def pin_bidir_unrolled(bidir):
    lengths, D, N = [13, 6], 5, 4
    off = np.concatenate([[0], np.cumsum(lengths)])
    T = int(off[-1])
    x, dt, Bm, Cm, A, Ds = _rand(21, T, D, N)
    _, dt2, Bm2, Cm2, A2, Ds2 = _rand(22, T, D, N)
    h0 = np.random.default_rng(23).standard_normal((2, D, N))
    rev = {"dt": dt2, "Bm": Bm2, "Cm": Cm2, "A": A2, "Dskip": Ds2}
    r = bidir(x, dt, Bm, Cm, A, Ds, rev=rev, seq_offsets=off, h_in=h0)
    for b in range(2):
        s = slice(off[b], off[b + 1])
        expect = _unrolled(x[s], dt[s], Bm[s], Cm[s], A, Ds, h0[b], False) + \
            _unrolled(x[s], dt2[s], Bm2[s], Cm2[s], A2, Ds2, np.zeros((D, N)), True)
        assert _rel(r["y"][s], expect) < 1e-12, (b, _rel(r["y"][s], expect))


def pin_bidir_flip(bidir):
    L, D, N = 15, 4, 5
    x, dt, Bm, Cm, A, Ds = _rand(24, L, D, N)
    _, dt2, Bm2, Cm2, A2, Ds2 = _rand(25, L, D, N)
    fl = lambda a: a[::-1].copy()
    r = bidir(x, dt, Bm, Cm, A, Ds, rev={"dt": dt2, "Bm": Bm2, "Cm": Cm2, "A": A2, "Dskip": Ds2},
              batch=1, seqlen=L)["y"]
    m = bidir(fl(x), fl(dt2), fl(Bm2), fl(Cm2), A2, Ds2,
              rev={"dt": fl(dt), "Bm": fl(Bm), "Cm": fl(Cm), "A": A, "Dskip": Ds},
              batch=1, seqlen=L)["y"]
    assert np.array_equal(r, fl(m))


def pin_bidir_gate(bidir):
    L, D = 8, 4
    x, dt, Bm, Cm, A, Ds = _rand(26, L, D, 3)
    res = np.random.default_rng(27).standard_normal((L, D))
    res[0, 0] = -0.0
    res[1, 1] = np.nan
    xx = x.copy()
    xx[3, 2] = np.inf          # y is inf or nan over the whole of channel 2
    r0 = bidir(xx, dt, Bm, Cm, A, Ds, batch=1, seqlen=L, res=res, s=0.0)
    assert np.array_equal(r0["out"].view(np.int64), res.view(np.int64))
    assert not np.any(np.isfinite(r0["y"][:, 2]))
    r1 = bidir(x, dt, Bm, Cm, A, Ds, batch=1, seqlen=L, res=res, s=-0.6)
    ok = ~np.isnan(res)
    assert np.array_equal(r1["out"][ok], (res + -0.6 * r1["y"])[ok])
    r2 = bidir(x, dt, Bm, Cm, A, Ds, batch=1, seqlen=L)
    assert np.array_equal(r2["out"], r2["y"])


BIDIR_PINS = [pin_bidir_direction_sums, pin_bidir_unrolled, pin_bidir_flip, pin_bidir_gate]
