"""The oracle against its committed regression fixture (CPU only)."""
import os

import numpy as np

from golden import make_golden

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _read(path):
    out, name, shape, vals = {}, None, None, []
    for line in open(path):
        if line.startswith("#"):
            continue
        parts = line.split()
        if len(parts) >= 2 and not parts[0][0].isdigit() and parts[0][0] not in "-+.n":
            if name:
                out[name] = np.array(vals, dtype=np.float64).reshape(shape)
            name, shape, vals = parts[0], tuple(int(p) for p in parts[1:]), []
        else:
            vals.append(float(parts[0]))
    out[name] = np.array(vals, dtype=np.float64).reshape(shape)
    return out


def test_oracle_matches_regression_fixture():
    stored = _read(os.path.join(HERE, "oracle_regression.txt"))
    now = make_golden.compute()
    assert set(stored) == set(now)
    for k in now:
        assert stored[k].shape == now[k].shape
        assert np.array_equal(stored[k], now[k]), k
