"""Pins that tie the fp64 oracle to something other than itself.

Each ``pin_*`` function takes ``scan``, a callable with the signature of
``oracle.selective_scan``, and raises ``AssertionError`` when the scan disagrees
with what the mathematics fixes. ``test_oracle_pins.py`` runs them against the
committed oracle; ``test_oracle_mutants.py`` runs them against builds of the
oracle with one planted mistake each and requires that some pin fails.

What pins what (the recurrence is the Mamba selective scan of the R2L stream in
"Bifocal Diffusion Language Models", section 2; the block/prefix split is from
"Training Hybrid Block Diffusion Language Models with Partial Bidirectionality",
"Methodology"):

* softplus              -- Delta against numpy's logaddexp(0, v) (a library routine)
* zero step             -- Delta = 0 keeps the state; y = C.h_in + Dskip.x (closed form)
* geometric series      -- constant inputs, closed form of the partial geometric sum
* suffix / prefix sums  -- A = 0, Delta = 1 reduces the scan to np.cumsum (exact)
* impulse               -- nothing leaks to the wrong side (exact zeros)
* unrolled form         -- the O(L^2 N) semiseparable sum built from cumulative
                           Delta sums, a different operation order, both directions,
                           with an initial state
* LTI                   -- constant Delta, B, C: a convolution (np.convolve)
* linearity             -- in x for fixed Delta, A, B, C
* flip                  -- reverse(x) == flip(forward(flip(x)))
* cache validity        -- prefix state then block commit == prefix state of the
                           whole; resumed forward readout == full readout on the tail
* tail block            -- reverse over the last block == full reverse, restricted
* chunked resume        -- reverse over the right part, state handed to the left part
* gate s                -- s = 0 returns the residual bit for bit (-0.0 and NaN in y
                           included); s != 0 gives res + s*y
"""
from __future__ import annotations

import numpy as np


def _rand(seed, tokens, D, N, dt_mean=-1.0):
    r = np.random.default_rng(seed)
    x = r.standard_normal((tokens, D))
    dt = r.normal(dt_mean, 0.7, (tokens, D))
    Bm = r.standard_normal((tokens, N))
    Cm = r.standard_normal((tokens, N))
    # A differs along both axes so that a transposed index shows
    A = -np.exp(r.normal(0.0, 0.5, (D, N))) * (1.0 + np.arange(N))[None, :]
    Dskip = r.standard_normal(D)
    return x, dt, Bm, Cm, A, Dskip


def _softplus_np(v):
    return np.logaddexp(0.0, v)


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# --------------------------------------------------------------------------
def pin_softplus(scan):
    x, dt, Bm, Cm, A, Ds = _rand(1, 24, 5, 4, dt_mean=0.0)
    dt = dt * 6.0  # spread over both branches of the stable form
    a = scan(x, dt, Bm, Cm, A, Ds, reverse=True, batch=1, seqlen=24, delta_softplus=True)["y"]
    b = scan(x, _softplus_np(dt), Bm, Cm, A, Ds, reverse=True, batch=1, seqlen=24,
             delta_softplus=False)["y"]
    assert _rel(a, b) < 1e-13, _rel(a, b)


def pin_zero_step(scan):
    x, dt, Bm, Cm, A, Ds = _rand(2, 12, 6, 4)
    dt[:] = 0.0
    for reverse in (True, False):
        r = scan(x, dt, Bm, Cm, A, Ds, reverse=reverse, batch=2, seqlen=6,
                 delta_softplus=False, want_h_out=True)
        assert np.array_equal(r["y"], Ds[None, :] * x)
        assert np.array_equal(r["h_out"], np.zeros((2, 6, 4)))
        h0 = np.random.default_rng(3).standard_normal((2, 6, 4))
        r = scan(x, dt, Bm, Cm, A, Ds, reverse=reverse, batch=2, seqlen=6,
                 delta_softplus=False, h_in=h0, want_h_out=True)
        assert np.array_equal(r["h_out"], h0)
        expect = np.concatenate([Cm[b * 6:(b + 1) * 6] @ h0[b].T for b in range(2)]) \
            + Ds[None, :] * x
        assert _rel(r["y"], expect) < 1e-14


def pin_geometric_series(scan):
    L, D, N = 40, 3, 5
    r = np.random.default_rng(4)
    delta = np.array([0.05, 0.3, 1.1])                      # per channel
    Bv, Cv = r.standard_normal(N), r.standard_normal(N)
    xv = r.standard_normal(D)
    A = -(np.arange(N) + 1.0)[None, :] * np.array([1.0, 0.5, 2.0])[:, None]
    Ds = r.standard_normal(D)
    x = np.tile(xv, (L, 1))
    dt = np.tile(delta, (L, 1))
    Bm, Cm = np.tile(Bv, (L, 1)), np.tile(Cv, (L, 1))
    a = np.exp(delta[:, None] * A)                          # [D, N]
    for reverse in (True, False):
        y = scan(x, dt, Bm, Cm, A, Ds, reverse=reverse, batch=1, seqlen=L,
                 delta_softplus=False)["y"]
        t = np.arange(L)
        m = (L - t) if reverse else (t + 1)                 # terms summed at position t
        h = (delta[None, :, None] * Bv[None, None, :] * xv[None, :, None]) \
            * (1.0 - a[None] ** m[:, None, None]) / (1.0 - a[None])
        expect = np.einsum("tdn,n->td", h, Cv) + Ds[None, :] * x
        assert _rel(y, expect) < 1e-12, _rel(y, expect)


def _unit_sum_inputs(lengths, D, N, seed):
    r = np.random.default_rng(seed)
    tokens = int(np.sum(lengths))
    x = r.integers(-8, 9, (tokens, D)).astype(np.float64)
    dt = np.ones((tokens, D))
    Bm = np.zeros((tokens, N))
    Cm = np.zeros((tokens, N))
    Bm[:, 0] = 1.0
    Cm[:, 0] = 1.0
    A = np.zeros((D, N))
    return x, dt, Bm, Cm, A


def pin_suffix_prefix_sums(scan):
    for lengths in ([9], [5, 0, 1, 7, 3], [0, 0, 2]):
        off = np.concatenate([[0], np.cumsum(lengths)])
        x, dt, Bm, Cm, A = _unit_sum_inputs(lengths, 4, 3, len(lengths))
        rev = scan(x, dt, Bm, Cm, A, None, reverse=True, seq_offsets=off,
                   delta_softplus=False, want_h_out=True)
        fwd = scan(x, dt, Bm, Cm, A, None, reverse=False, seq_offsets=off,
                   delta_softplus=False, want_h_out=True)
        for b in range(len(lengths)):
            seg = slice(off[b], off[b + 1])
            xs = x[seg]
            assert np.array_equal(rev["y"][seg], np.cumsum(xs[::-1], axis=0)[::-1])
            assert np.array_equal(fwd["y"][seg], np.cumsum(xs, axis=0))
            total = xs.sum(axis=0)
            assert np.array_equal(rev["h_out"][b, :, 0], total)
            assert np.array_equal(fwd["h_out"][b, :, 0], total)
            assert not np.any(rev["h_out"][b, :, 1:])


def pin_impulse(scan):
    L, t0 = 16, 6
    x, dt, Bm, Cm, A, Ds = _rand(5, L, 4, 3)
    x[:] = 0.0
    x[t0] = np.random.default_rng(6).standard_normal(4)
    rev = scan(x, dt, Bm, Cm, A, Ds, reverse=True, batch=1, seqlen=L)["y"]
    fwd = scan(x, dt, Bm, Cm, A, Ds, reverse=False, batch=1, seqlen=L)["y"]
    assert np.all(rev[t0 + 1:] == 0.0) and np.all(rev[:t0 + 1] != 0.0)
    assert np.all(fwd[:t0] == 0.0) and np.all(fwd[t0:] != 0.0)


def _unrolled(x, dt, Bm, Cm, A, Ds, h_in, reverse):
    """y from the semiseparable sum over pairs of tokens (one sequence)."""
    L = x.shape[0]
    delta = _softplus_np(dt)                                # [L, D]
    cs = np.concatenate([np.zeros((1, x.shape[1])), np.cumsum(delta, axis=0)])  # [L+1, D]
    u = delta[:, :, None] * Bm[:, None, :] * x[:, :, None]  # [L, D, N] input of token tau
    y = np.zeros_like(x)
    for t in range(L):
        if reverse:
            taus = np.arange(t, L)
            seg = cs[taus] - cs[t]                          # sum_{k=t}^{tau-1} delta_k
            tail = cs[L] - cs[t]                            # sum_{k=t}^{L-1}
        else:
            taus = np.arange(0, t + 1)
            seg = cs[t + 1] - cs[taus + 1]                  # sum_{k=tau+1}^{t} delta_k
            tail = cs[t + 1] - cs[0]                        # sum_{k=0}^{t}
        dec = np.exp(seg[:, :, None] * A[None])             # [taus, D, N]
        h = np.sum(dec * u[taus], axis=0) + np.exp(tail[:, None] * A) * h_in
        y[t] = h @ Cm[t] + Ds * x[t]
    return y


def pin_unrolled(scan):
    L, D, N = 13, 5, 4
    x, dt, Bm, Cm, A, Ds = _rand(7, L, D, N)
    h0 = np.random.default_rng(8).standard_normal((1, D, N))
    for reverse in (True, False):
        y = scan(x, dt, Bm, Cm, A, Ds, reverse=reverse, batch=1, seqlen=L, h_in=h0)["y"]
        expect = _unrolled(x, dt, Bm, Cm, A, Ds, h0[0], reverse)
        assert _rel(y, expect) < 1e-12, (reverse, _rel(y, expect))


def pin_lti(scan):
    L, N = 50, 6
    r = np.random.default_rng(9)
    delta = 0.2
    Bv, Cv = r.standard_normal(N), r.standard_normal(N)
    A = -(np.arange(N) + 1.0)[None, :] * 0.7
    x = r.standard_normal((L, 1))
    ds = np.array([0.3])
    a = np.exp(delta * A[0])
    K = np.array([np.sum(Cv * a ** k * delta * Bv) for k in range(L)])
    y = scan(x, np.full((L, 1), delta), np.tile(Bv, (L, 1)), np.tile(Cv, (L, 1)), A, ds,
             reverse=True, batch=1, seqlen=L, delta_softplus=False)["y"][:, 0]
    expect = np.convolve(x[::-1, 0], K)[:L][::-1] + ds[0] * x[:, 0]
    assert _rel(y, expect) < 1e-12, _rel(y, expect)


def pin_linearity(scan):
    x1, dt, Bm, Cm, A, Ds = _rand(10, 20, 3, 4)
    x2 = np.random.default_rng(11).standard_normal(x1.shape)
    al, be = 0.75, -1.5
    f = lambda x: scan(x, dt, Bm, Cm, A, Ds, reverse=True, batch=2, seqlen=10)["y"]
    assert _rel(f(al * x1 + be * x2), al * f(x1) + be * f(x2)) < 1e-12


def pin_flip(scan):
    L = 15
    x, dt, Bm, Cm, A, Ds = _rand(12, L, 4, 5)
    h0 = np.random.default_rng(13).standard_normal((1, 4, 5))
    rev = scan(x, dt, Bm, Cm, A, Ds, reverse=True, batch=1, seqlen=L, h_in=h0, want_h_out=True)
    fl = lambda a: a[::-1].copy()
    fwd = scan(fl(x), fl(dt), fl(Bm), fl(Cm), A, Ds, reverse=False, batch=1, seqlen=L,
               h_in=h0, want_h_out=True)
    assert np.array_equal(rev["y"], fl(fwd["y"]))
    assert np.array_equal(rev["h_out"], fwd["h_out"])


def pin_cache_validity(scan):
    P, T, D, N = 11, 6, 4, 3
    x, dt, Bm, Cm, A, Ds = _rand(14, P + T, D, N)
    full = scan(x, dt, Bm, Cm, A, Ds, reverse=False, batch=1, seqlen=P + T, want_h_out=True)
    pre = scan(x[:P], dt[:P], Bm[:P], None, A, None, reverse=False, batch=1, seqlen=P,
               want_y=False, want_h_out=True)["h_out"]
    com = scan(x[P:], dt[P:], Bm[P:], Cm[P:], A, Ds, reverse=False, batch=1, seqlen=T,
               h_in=pre, want_h_out=True)
    assert np.array_equal(com["h_out"], full["h_out"])
    assert np.array_equal(com["y"], full["y"][P:])


def pin_tail_block(scan):
    P, T = 9, 5
    x, dt, Bm, Cm, A, Ds = _rand(15, P + T, 3, 4)
    full = scan(x, dt, Bm, Cm, A, Ds, reverse=True, batch=1, seqlen=P + T)["y"]
    blk = scan(x[P:], dt[P:], Bm[P:], Cm[P:], A, Ds, reverse=True, batch=1, seqlen=T)["y"]
    assert np.array_equal(blk, full[P:])


def pin_chunked_resume(scan):
    L, cut = 17, 7
    x, dt, Bm, Cm, A, Ds = _rand(16, L, 3, 4)
    full = scan(x, dt, Bm, Cm, A, Ds, reverse=True, batch=1, seqlen=L, want_h_out=True)
    right = scan(x[cut:], dt[cut:], Bm[cut:], Cm[cut:], A, Ds, reverse=True, batch=1,
                 seqlen=L - cut, want_h_out=True)
    left = scan(x[:cut], dt[:cut], Bm[:cut], Cm[:cut], A, Ds, reverse=True, batch=1,
                seqlen=cut, h_in=right["h_out"], want_h_out=True)
    assert np.array_equal(np.concatenate([left["y"], right["y"]]), full["y"])
    assert np.array_equal(left["h_out"], full["h_out"])


def pin_gate(scan):
    L = 8
    x, dt, Bm, Cm, A, Ds = _rand(17, L, 4, 3)
    res = np.random.default_rng(18).standard_normal((L, 4))
    res[0, 0] = -0.0
    res[1, 1] = np.nan
    xx = x.copy()
    xx[3, 2] = np.inf          # y turns inf / nan from here leftwards in channel 2
    r0 = scan(xx, dt, Bm, Cm, A, Ds, reverse=True, batch=1, seqlen=L, res=res, s=0.0,
              want_out=True)
    assert np.array_equal(r0["out"].view(np.int64), res.view(np.int64))
    assert not np.all(np.isfinite(r0["y"]))
    r1 = scan(x, dt, Bm, Cm, A, Ds, reverse=True, batch=1, seqlen=L, res=res, s=0.37,
              want_out=True)
    expect = res + 0.37 * r1["y"]
    ok = ~np.isnan(res)
    assert np.array_equal(r1["out"][ok], expect[ok])
    r2 = scan(x, dt, Bm, Cm, A, Ds, reverse=True, batch=1, seqlen=L, want_out=True)
    assert np.array_equal(r2["out"], r2["y"])


PINS = [pin_softplus, pin_zero_step, pin_geometric_series, pin_suffix_prefix_sums,
        pin_impulse, pin_unrolled, pin_lti, pin_linearity, pin_flip, pin_cache_validity,
        pin_tail_block, pin_chunked_resume, pin_gate]
