"""Pins that tie the oracle's backward (``oracle.selective_scan_backward``) to
something other than itself.

Each ``pin_*`` takes ``bwd`` (a callable with the signature of
``oracle.selective_scan_backward``) and raises ``AssertionError`` on a
disagreement. ``test_oracle_pins.py`` runs them on the committed oracle;
``test_oracle_mutants.py`` on builds with one planted mistake each in the
backward, and requires that some pin fails.

The loss is L = sum(dout * out) + sum(dh_out * h_out) for the scan of the R2L
stream ("Bifocal Diffusion Language Models", section 2: reverse selective scan,
residual through the gate s), whose sidecar the pages train.

* finite differences -- central differences of the forward oracle (itself pinned
                        by ``oracle_pins``), for every input element and s,
                        every residual form and both directions
* autograd           -- torch.autograd in float64 through a plain torch loop
                        written here (a library routine for the derivative)
* prefix sums        -- A = 0, Delta = 1, B = C = e_0: the forward is a suffix
                        sum, whose adjoint is the prefix sum of dout (exact)
* linearity          -- the gradients are linear in (dout, dh_out)
"""
from __future__ import annotations

import numpy as np

import oracle


def _inputs(seed, lengths, D, N):
    r = np.random.default_rng(seed)
    T = int(sum(lengths))
    x = r.standard_normal((T, D))
    dt = r.normal(-0.5, 0.8, (T, D))
    Bm = r.standard_normal((T, N))
    Cm = r.standard_normal((T, N))
    A = -np.exp(r.normal(0.0, 0.5, (D, N))) * (1.0 + np.arange(N))[None, :]
    Dskip = r.standard_normal(D)
    h_in = r.standard_normal((len(lengths), D, N))
    dout = r.standard_normal((T, D))
    dh_out = r.standard_normal((len(lengths), D, N))
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    return dict(x=x, dt=dt, Bm=Bm, Cm=Cm, A=A, Dskip=Dskip, h_in=h_in), dout, dh_out, off


def _loss(v, off, reverse, res_kind, s, dout, dh_out, softplus=True):
    res = {"none": None, "x": v["x"], "separate": v["res"]}[res_kind]
    r = oracle.selective_scan(v["x"], v["dt"], v["Bm"], v["Cm"], v["A"], v["Dskip"],
                              reverse=reverse, seq_offsets=off, h_in=v["h_in"],
                              want_h_out=True, want_y=False, want_out=True, res=res, s=s,
                              delta_softplus=softplus)
    return float(np.sum(dout * r["out"]) + np.sum(dh_out * r["h_out"]))


def _rel(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b))) /
                 max(float(np.max(np.abs(np.asarray(b)))), 1e-300))


def pin_bwd_finite_differences(bwd):
    lengths, D, N = [4, 0, 3], 3, 4
    eps = 1e-6
    for reverse in (True, False):
        for res_kind, s in (("none", 0.0), ("x", 0.7), ("separate", -0.4)):
            for softplus in ((True, False) if res_kind == "none" else (True,)):
                v, dout, dh_out, off = _inputs(11, lengths, D, N)
                v["res"] = np.random.default_rng(12).standard_normal(v["x"].shape)
                if not softplus:   # Delta = dt directly: keep it positive (decaying states)
                    v["dt"] = np.abs(v["dt"]) + 0.05
                g = bwd(v["x"], v["dt"], v["Bm"], v["Cm"], v["A"], v["Dskip"], reverse=reverse,
                        dout=dout, dh_out=dh_out, res_kind=res_kind, s=s, seq_offsets=off,
                        h_in=v["h_in"], delta_softplus=softplus)
                for name, gname in (("x", "dx"), ("dt", "ddt"), ("Bm", "dBm"), ("Cm", "dCm"),
                                    ("A", "dA"), ("Dskip", "dDskip"), ("h_in", "dh_in")):
                    num = np.zeros_like(v[name])
                    for idx in np.ndindex(v[name].shape):
                        keep = v[name][idx]
                        v[name][idx] = keep + eps
                        lp = _loss(v, off, reverse, res_kind, s, dout, dh_out, softplus)
                        v[name][idx] = keep - eps
                        lm = _loss(v, off, reverse, res_kind, s, dout, dh_out, softplus)
                        v[name][idx] = keep
                        num[idx] = (lp - lm) / (2 * eps)
                    e = _rel(g[gname], num)
                    assert e < 1e-6, "d%s (reverse=%s, res=%s, softplus=%s): %.2e" % (
                        name, reverse, res_kind, softplus, e)
                if res_kind != "none":
                    num = (_loss(v, off, reverse, res_kind, s + eps, dout, dh_out) -
                           _loss(v, off, reverse, res_kind, s - eps, dout, dh_out)) / (2 * eps)
                    assert abs(g["ds"] - num) <= 1e-6 * max(abs(num), 1.0), (g["ds"], num)


def _torch_scan(x, dt, Bm, Cm, A, Dskip, h_in, off, reverse, s, res_kind, res):
    """The forward, written as a plain torch loop (float64) for autograd."""
    import torch
    outs, hs = [], []
    for b in range(len(off) - 1):
        h = h_in[b]
        rows = list(range(int(off[b]), int(off[b + 1])))
        seq = [None] * len(rows)
        for t in (reversed(rows) if reverse else rows):
            delta = torch.nn.functional.softplus(dt[t])               # [D]
            a = torch.exp(delta[:, None] * A)                          # [D, N]
            h = a * h + (delta * x[t])[:, None] * Bm[t][None, :]
            y = h @ Cm[t] + Dskip * x[t]
            seq[t - int(off[b])] = y if res_kind == "none" else \
                (x[t] if res_kind == "x" else res[t]) + s * y
        outs += seq
        hs.append(h)
    return torch.stack(outs), torch.stack(hs)


def pin_bwd_autograd(bwd):
    import torch
    lengths, D, N = [9, 1, 0, 6], 5, 16
    for reverse, res_kind, s in ((True, "x", 0.3), (False, "none", 0.0), (True, "separate", 1.2)):
        v, dout, dh_out, off = _inputs(13, lengths, D, N)
        res = np.random.default_rng(14).standard_normal(v["x"].shape)
        tv = {k: torch.tensor(a, dtype=torch.float64, requires_grad=True) for k, a in v.items()}
        ts = torch.tensor(s, dtype=torch.float64, requires_grad=True)
        out, h = _torch_scan(tv["x"], tv["dt"], tv["Bm"], tv["Cm"], tv["A"], tv["Dskip"],
                             tv["h_in"], off, reverse, ts, res_kind, torch.tensor(res))
        loss = (out * torch.tensor(dout)).sum() + (h * torch.tensor(dh_out)).sum()
        loss.backward()
        g = bwd(v["x"], v["dt"], v["Bm"], v["Cm"], v["A"], v["Dskip"], reverse=reverse,
                dout=dout, dh_out=dh_out, res_kind=res_kind, s=s, seq_offsets=off,
                h_in=v["h_in"])
        for name, gname in (("x", "dx"), ("dt", "ddt"), ("Bm", "dBm"), ("Cm", "dCm"),
                            ("A", "dA"), ("Dskip", "dDskip"), ("h_in", "dh_in")):
            e = _rel(g[gname], tv[name].grad.numpy())
            assert e < 1e-12, "autograd d%s (reverse=%s, res=%s): %.2e" % (name, reverse,
                                                                           res_kind, e)
        if res_kind != "none":
            assert abs(g["ds"] - ts.grad.item()) <= 1e-12 * max(abs(ts.grad.item()), 1.0)


def pin_bwd_prefix_sums(bwd):
    """A = 0, Delta = 1, B = C = e_0, Dskip = 0: the reverse scan outputs suffix
    sums of x, so dL/dx is the prefix sum of dout (forward: the other way)."""
    lengths, D, N = [7, 1, 0, 5], 3, 16
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    T = int(off[-1])
    r = np.random.default_rng(15)
    x = r.integers(-4, 5, (T, D)).astype(np.float64)
    dout = r.integers(-4, 5, (T, D)).astype(np.float64)
    Bm = np.zeros((T, N))
    Bm[:, 0] = 1.0
    for reverse in (True, False):
        g = bwd(x, np.ones((T, D)), Bm, Bm.copy(), np.zeros((D, N)), np.zeros(D),
                reverse=reverse, dout=dout, seq_offsets=off, delta_softplus=False)
        want = np.zeros((T, D))
        for b in range(len(lengths)):
            seg = dout[off[b]:off[b + 1]]
            want[off[b]:off[b + 1]] = np.cumsum(seg, axis=0) if reverse else \
                np.cumsum(seg[::-1], axis=0)[::-1]
        assert np.array_equal(g["dx"], want), "prefix-sum adjoint (reverse=%s)" % reverse


def pin_bwd_linearity(bwd):
    lengths, D, N = [6, 4], 4, 8
    v, d1, h1, off = _inputs(16, lengths, D, N)
    _, d2, h2, _ = _inputs(17, lengths, D, N)
    kw = dict(reverse=True, seq_offsets=off, h_in=v["h_in"], res_kind="x", s=0.6)
    args = (v["x"], v["dt"], v["Bm"], v["Cm"], v["A"], v["Dskip"])
    ga = bwd(*args, dout=d1, dh_out=h1, **kw)
    gb = bwd(*args, dout=d2, dh_out=h2, **kw)
    gc = bwd(*args, dout=2.0 * d1 - 3.0 * d2, dh_out=2.0 * h1 - 3.0 * h2, **kw)
    for k in ("dx", "ddt", "dBm", "dCm", "dA", "dDskip", "dh_in", "ds"):
        want = 2.0 * np.asarray(ga[k]) - 3.0 * np.asarray(gb[k])
        assert _rel(gc[k], want) < 1e-12, "linearity " + k


BWD_PINS = [pin_bwd_finite_differences, pin_bwd_autograd, pin_bwd_prefix_sums, pin_bwd_linearity]
