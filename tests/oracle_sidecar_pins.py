"""Pins of the oracle's sidecar block (``oracle.sidecar_forward``).

Each ``pin_*`` takes ``sidecar``, a callable with the signature of
``oracle.sidecar_forward``, and raises ``AssertionError`` when it disagrees
with what fixes it independently:

* causal block, flipped -- the pages define the R2L stream as: reverse the
  sequence, run the Mamba block, reverse back. A causal Mamba block written
  here with torch float64 ops (F.linear, a left-padded F.conv1d, SiLU, a plain
  recurrence loop) run on each flipped sequence and flipped back must give the
  oracle's output (tap order, which half gates, dt bias, B/C columns,
  projection orientation and direction all enter)
* gate          -- s = 0 returns hidden bit for bit; s != 0 is linear in s
* zero out-projection -- W_out = 0 leaves hidden unchanged
* storage rounding -- with store="bf16" every stored intermediate is a bf16
  value, and the result stays within bf16 error of the unrounded one
"""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F


def _weights(seed, dm, di, R, N, K):
    r = np.random.default_rng(seed)
    W_in = r.standard_normal((2 * di, dm)) / np.sqrt(dm)
    conv_w = r.standard_normal((di, K)) * 0.5
    conv_b = r.standard_normal(di) * 0.1
    W_x = r.standard_normal((R + 2 * N, di)) / np.sqrt(di)
    W_dt = r.standard_normal((di, R)) / np.sqrt(R)
    dt_bias = r.normal(-1.0, 0.3, di)
    A = -np.exp(r.normal(0.0, 0.5, (di, N))) * (1.0 + np.arange(N))[None, :]
    Dskip = r.standard_normal(di)
    W_out = r.standard_normal((dm, di)) / np.sqrt(di)
    return W_in, conv_w, conv_b, W_x, W_dt, dt_bias, A, Dskip, W_out


def _causal_block(h, W_in, conv_w, conv_b, W_x, W_dt, dt_bias, A, Dskip, W_out):
    """A left-to-right Mamba block on one sequence, float64 torch (no residual)."""
    t = lambda a: torch.as_tensor(a, dtype=torch.float64)   # noqa: E731
    h = t(h)
    di, R, N, K = W_dt.shape[0], W_dt.shape[1], A.shape[1], conv_w.shape[1]
    xz = F.linear(h, t(W_in))
    x, z = xz[:, :di], xz[:, di:]
    L = x.shape[0]
    c = F.conv1d(x.T[None], t(conv_w)[:, None, :], t(conv_b), padding=K - 1, groups=di)
    u = F.silu(c[0, :, :L].T)
    xdbl = F.linear(u, t(W_x))
    dt = F.linear(xdbl[:, :R], t(W_dt)) + t(dt_bias)
    delta = F.softplus(dt)
    Bm, Cm = xdbl[:, R:R + N], xdbl[:, R + N:]
    hs = torch.zeros(di, N, dtype=torch.float64)
    ys = []
    for k in range(L):
        hs = torch.exp(delta[k][:, None] * t(A)) * hs + (delta[k] * u[k])[:, None] * Bm[k][None, :]
        ys.append(hs @ Cm[k] + t(Dskip) * u[k])
    y = torch.stack(ys) if ys else torch.zeros(0, di, dtype=torch.float64)
    return F.linear(y * F.silu(z), t(W_out)).numpy()


def pin_sidecar_causal_block_flipped(sidecar):
    dm, di, R, N, K = 6, 8, 3, 4, 4
    lengths = [9, 1, 0, 5]
    off = np.concatenate([[0], np.cumsum(lengths)])
    w = _weights(61, dm, di, R, N, K)
    hidden = np.random.default_rng(62).standard_normal((int(off[-1]), dm))
    s = 0.7
    got = sidecar(hidden, *w, s=s, seq_offsets=off)["out"]
    for b in range(len(lengths)):
        sl = slice(off[b], off[b + 1])
        if off[b + 1] == off[b]:
            continue
        o = _causal_block(hidden[sl][::-1].copy(), *w)[::-1]
        expect = hidden[sl] + s * o
        err = np.max(np.abs(got[sl] - expect)) / np.max(np.abs(expect))
        assert err < 1e-12, (b, err)


def pin_sidecar_gate(sidecar):
    dm, di, R, N, K = 5, 6, 2, 3, 3
    w = _weights(63, dm, di, R, N, K)
    hidden = np.random.default_rng(64).standard_normal((7, dm))
    hidden[0, 0] = -0.0
    hidden[1, 1] = np.nan
    r0 = sidecar(hidden, *w, s=0.0, batch=1, seqlen=7)["out"]
    assert np.array_equal(r0.view(np.int64), hidden.view(np.int64))
    h2 = np.random.default_rng(65).standard_normal((7, dm))
    a = sidecar(h2, *w, s=0.25, batch=1, seqlen=7)["out"] - h2
    b = sidecar(h2, *w, s=-0.5, batch=1, seqlen=7)["out"] - h2
    assert np.max(np.abs(b + 2.0 * a)) <= 1e-12 * np.max(np.abs(a))


def pin_sidecar_zero_out_projection(sidecar):
    dm, di, R, N, K = 5, 6, 2, 3, 4
    w = list(_weights(66, dm, di, R, N, K))
    w[-1] = np.zeros_like(w[-1])
    hidden = np.random.default_rng(67).standard_normal((10, dm))
    r = sidecar(hidden, *w, s=0.9, batch=2, seqlen=5)
    assert np.array_equal(r["out"], hidden)
    assert np.any(r["g"] != 0.0)


def pin_sidecar_storage_rounding(sidecar):
    dm, di, R, N, K = 8, 16, 4, 4, 4
    w = _weights(68, dm, di, R, N, K)
    hidden = np.random.default_rng(69).standard_normal((12, dm))
    exact = sidecar(hidden, *w, s=1.0, batch=2, seqlen=6)
    r = sidecar(hidden, *w, s=1.0, batch=2, seqlen=6, store="bf16")
    for k in ("xz", "u", "xdbl", "g"):
        v = r[k].astype(np.float32)
        assert np.array_equal(v.astype(np.float64), r[k]), k          # fp32 values...
        assert not np.any(v.view(np.uint32) & 0xFFFF), k                # ... with bf16 bits only
    err = np.max(np.abs(r["out"] - exact["out"])) / np.max(np.abs(exact["out"]))
    assert 0.0 < err < 2e-2, err


SIDECAR_PINS = [pin_sidecar_causal_block_flipped, pin_sidecar_gate,
                pin_sidecar_zero_out_projection, pin_sidecar_storage_rounding]
