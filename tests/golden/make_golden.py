"""Writes the oracle regression fixture ``oracle_regression.txt``.

The pages print no worked numeric example for the scan, so this directory holds
no value taken from them. The fixture below is written by the committed oracle
alone (plus the seeded inputs of ``synth``); it pins the oracle to its own past
output so that any later change of its arithmetic shows up as a failing test
and has to be justified. Run from the repo root: ``python tests/golden/make_golden.py``.
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

KEY = 7
LENGTHS = [5, 11, 0, 3]
D, N = 6, 16
S = 0.25


def compute():
    inp = synth.scan_inputs(KEY, LENGTHS, D=D, N=N, dtype="f32")
    h0 = synth.initial_state(KEY, len(LENGTHS), D, N, scale=0.5)
    rev = oracle.r2l_scan(inp.x, inp.dt, inp.Bm, inp.Cm, inp.A, inp.Dskip, res=inp.x, s=S,
                          seq_offsets=inp.offsets, h_in=h0, want_h_out=True)
    fwd = oracle.selective_scan(inp.x, inp.dt, inp.Bm, None, inp.A, None, reverse=False,
                                seq_offsets=inp.offsets, h_in=h0, want_y=False,
                                want_h_out=True)
    vals = {"r2l_y": rev["y"], "r2l_out": rev["out"], "r2l_h_out": rev["h_out"],
            "fwd_h_out": fwd["h_out"]}
    # the bidirectional scan, reverse parameters of its own
    rv = synth.reverse_params(KEY, LENGTHS, D, N=N)
    bi = oracle.bidir_scan(inp.x, inp.dt, inp.Bm, inp.Cm, inp.A, inp.Dskip, rev=rv,
                           seq_offsets=inp.offsets, h_in=h0, res=inp.x, s=S, want_h_out=True)
    vals.update(bidir_y=bi["y"], bidir_out=bi["out"], bidir_h_out=bi["h_out"])
    # the backward of the R2L scan (res = x) for a seeded dL/dout and dL/dh_out
    r = np.random.default_rng(KEY)
    g = oracle.selective_scan_backward(
        inp.x, inp.dt, inp.Bm, inp.Cm, inp.A, inp.Dskip, reverse=True,
        dout=r.standard_normal(inp.x.shape), dh_out=r.standard_normal(h0.shape), res_kind="x",
        s=S, seq_offsets=inp.offsets, h_in=h0)
    for k in ("dx", "ddt", "dBm", "dCm", "dA", "dDskip", "dh_in"):
        vals["bwd_" + k] = g[k]
    vals["bwd_ds"] = np.array([g["ds"]])
    # the sidecar block at small widths (d_model 8, d_inner 16, dt_rank 8)
    w = synth.sidecar_weights(KEY, 8, 16, 8, N=N)
    hid = synth.hidden_states(KEY, LENGTHS, 8)
    sc = oracle.sidecar_forward(hid, w["W_in"], w["conv_w"], w["conv_b"], w["W_x"], w["W_dt"],
                                w["dt_bias"], w["A"], w["Dskip"], w["W_out"], s=S,
                                seq_offsets=inp.offsets)
    vals.update(sidecar_out=sc["out"], sidecar_y=sc["y"])
    return vals


def main():
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_regression.txt")
    vals = compute()
    with open(path, "w") as f:
        f.write("# oracle regression fixture: synth.scan_inputs(key=%d, lengths=%s, D=%d, "
                "N=%d, f32), h_in = synth.initial_state(key, 4, D, N, 0.5), res = x, s = %r\n"
                % (KEY, LENGTHS, D, N, S))
        f.write("# bidir: synth.reverse_params(key, lengths, D); backward: dout, dh_out ~ "
                "numpy default_rng(key); sidecar: synth.sidecar_weights(key, 8, 16, 8), "
                "synth.hidden_states(key, lengths, 8)\n")
        f.write("# written by tests/golden/make_golden.py from oracle/ only\n")
        for name, arr in vals.items():
            flat = arr.reshape(-1)
            f.write("%s %s\n" % (name, " ".join(str(v) for v in arr.shape)))
            for v in flat:
                f.write("%.17g\n" % v)


if __name__ == "__main__":
    main()
