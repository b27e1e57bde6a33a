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
    return {"r2l_y": rev["y"], "r2l_out": rev["out"], "r2l_h_out": rev["h_out"],
            "fwd_h_out": fwd["h_out"]}


def main():
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_regression.txt")
    vals = compute()
    with open(path, "w") as f:
        f.write("# oracle regression fixture: synth.scan_inputs(key=%d, lengths=%s, D=%d, "
                "N=%d, f32), h_in = synth.initial_state(key, 4, D, N, 0.5), res = x, s = %r\n"
                % (KEY, LENGTHS, D, N, S))
        f.write("# written by tests/golden/make_golden.py from oracle/ only\n")
        for name, arr in vals.items():
            flat = arr.reshape(-1)
            f.write("%s %s\n" % (name, " ".join(str(v) for v in arr.shape)))
            for v in flat:
                f.write("%.17g\n" % v)


if __name__ == "__main__":
    main()
