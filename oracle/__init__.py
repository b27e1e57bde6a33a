"""fp64 CPU oracle for the R2L / forward selective scans -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg
may import this package. The product (``reverse_mamba_selective_amd``) never
imports it, and it never imports the product: the two share no code. The only
common module is ``synth`` (seeded random inputs, no arithmetic of the method).

The arithmetic lives in ``selective_scan_ref.c`` (plain fp64 loops; see its
header for the passages of "Bifocal Diffusion Language Models" and "Training
Hybrid Block Diffusion Language Models with Partial Bidirectionality" that it
follows). This module only builds that file with gcc, marshals numpy arrays to
contiguous fp64 and calls it.

Function map (each a thin wrapper over the one C routine):

* ``selective_scan``      -- the general routine (either direction, optional
                             state in/out, readout, gated residual).
* ``r2l_scan``            -- the R2L stream: reverse scan, readout, optional
                             residual ``res + s * y`` (nl/fr summaries, section 2).
* ``prefix_scan_state``   -- forward-only boundary state of each prefix
                             (partial-bidirectionality summary, "Methodology" 1).
* ``block_commit_state``  -- advance a cached boundary state over a committed
                             block (same passage: finished blocks join the prefix).
* ``bidir_scan``          -- forward plus reverse scan of the same x, each with
                             its own parameters, readouts added (the full-window
                             bidirectional scan of the earlier hybrids).
* ``sidecar_forward``     -- the sidecar block around the reverse scan (a reading:
                             the Mamba block's projections, conv and gate; numpy
                             matmuls plus the C scan).
* ``selective_scan_backward`` -- the gradients of the scan with readout and
                             residual (training the R2L stream).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import time

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "selective_scan_ref.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_SAN_PATH = os.path.join(_HERE, "_san", "liboracle.so")
_lib = None

_dptr = ctypes.POINTER(ctypes.c_double)
_i64ptr = ctypes.POINTER(ctypes.c_int64)


def build(force: bool = True, src: str = _SRC, out: str = _LIB_PATH, sanitize: bool = False) -> str:
    """Compile the oracle with gcc (fp64, no fast-math, no FMA contraction).
    sanitize: a copy under oracle/_san/ built by ROCm's clang with
    AddressSanitizer and UndefinedBehaviorSanitizer (no OpenMP), to run with the
    sanitized library of the scan (whose sanitizer runtime it shares)."""
    if sanitize:
        out = _SAN_PATH
        os.makedirs(os.path.dirname(out), exist_ok=True)
    elif not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(src):
        return out
    tmp = out + ".tmp%d" % os.getpid()
    if sanitize:
        clang = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", "clang")
        cmd = [clang, "-O1", "-g", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off",
               "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
               "-fno-omit-frame-pointer", "-shared-libsan", "-Wno-unknown-pragmas",
               "-o", tmp, src, "-lm"]
    else:
        cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
               "-ffp-contract=off", "-fno-fast-math", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


class OracleLib:
    """ctypes view of one build of selective_scan_ref.c."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        lib.ref_selective_scan.restype = ctypes.c_int
        lib.ref_selective_scan.argtypes = [
            ctypes.c_int, ctypes.c_int64, _i64ptr, ctypes.c_int64, ctypes.c_int64,
            _dptr, _dptr, _dptr, _dptr, _dptr, _dptr, ctypes.c_int,
            _dptr, _dptr, _dptr, _dptr, ctypes.c_double, _dptr, ctypes.c_int]
        lib.ref_max_threads.restype = ctypes.c_int
        lib.ref_max_threads.argtypes = []
        if hasattr(lib, "ref_selective_scan_backward"):
            lib.ref_selective_scan_backward.restype = ctypes.c_int
            lib.ref_selective_scan_backward.argtypes = [
                ctypes.c_int, ctypes.c_int64, _i64ptr, ctypes.c_int64, ctypes.c_int64,
                _dptr, _dptr, _dptr, _dptr, _dptr, _dptr, ctypes.c_int, _dptr,
                ctypes.c_int, ctypes.c_double, _dptr, _dptr,
                _dptr, _dptr, _dptr, _dptr, _dptr, _dptr, _dptr, _dptr, ctypes.c_int]
        if hasattr(lib, "ref_bidir_scan"):
            lib.ref_bidir_scan.restype = ctypes.c_int
            lib.ref_bidir_scan.argtypes = [
                ctypes.c_int64, _i64ptr, ctypes.c_int64, ctypes.c_int64, _dptr,
                _dptr, _dptr, _dptr, _dptr, _dptr, _dptr, _dptr, _dptr, _dptr, _dptr,
                ctypes.c_int, _dptr, _dptr, _dptr, _dptr, ctypes.c_double, _dptr, ctypes.c_int]
        self.lib = lib
        self.path = path


def _load() -> OracleLib:
    global _lib
    if _lib is None:
        alt = os.environ.get("R2L_ORACLE_LIB")   # another build (the sanitized one)
        if alt:
            _lib = OracleLib(alt)
            return _lib
        if not os.path.exists(_LIB_PATH) or \
                os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        _lib = OracleLib(_LIB_PATH)
    return _lib


def max_threads() -> int:
    return int(_load().lib.ref_max_threads())


def _f64(a):
    if a is None:
        return None
    if hasattr(a, "detach"):  # a CPU torch tensor (bf16 is widened exactly)
        import torch
        a = a.detach().to("cpu", torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_dptr)


def _offsets(seq_offsets, batch, seqlen, tokens):
    if seq_offsets is None:
        if batch is None or seqlen is None:
            raise ValueError("dense layout needs batch and seqlen")
        off = np.arange(batch + 1, dtype=np.int64) * int(seqlen)
    else:
        off = np.ascontiguousarray(np.asarray(seq_offsets, dtype=np.int64))
    if off[-1] != tokens:
        raise ValueError("offsets end at %d but there are %d tokens" % (off[-1], tokens))
    return off


def selective_scan(x, dt, Bm, Cm, A, Dskip=None, *, reverse: bool,
                   seq_offsets=None, batch=None, seqlen=None,
                   delta_softplus: bool = True, h_in=None, want_h_out=False,
                   want_y=True, res=None, s: float = 0.0, want_out=False,
                   nthreads: int = 0, timing: dict | None = None,
                   lib: OracleLib | None = None):
    """Run the fp64 scan. x, dt: [tokens, D]; Bm, Cm: [tokens, N]; A: [D, N].

    Returns a dict with fp64 numpy arrays ``y`` [tokens, D], ``out``
    [tokens, D] and ``h_out`` [batch, D, N] as requested. If ``timing`` is a
    dict, the wall time of the C call alone is stored under ``"seconds"``.
    ``lib`` selects another build of the same source (the default is the
    committed one).
    """
    x = _f64(x)
    dt = _f64(dt)
    Bm = _f64(Bm)
    Cm = _f64(Cm)
    A = _f64(A)
    Dskip = _f64(Dskip)
    h_in = _f64(h_in)
    res = _f64(res)
    tokens, D = x.shape
    N = A.shape[1]
    off = _offsets(seq_offsets, batch, seqlen, tokens)
    nb = off.shape[0] - 1
    assert dt.shape == (tokens, D) and Bm.shape == (tokens, N) and A.shape == (D, N)
    if Cm is not None:
        assert Cm.shape == (tokens, N)
    if Dskip is not None:
        assert Dskip.shape == (D,)
    if h_in is not None:
        h_in = h_in.reshape(nb, D, N)
    if res is not None:
        assert res.shape == (tokens, D)
    y = np.empty((tokens, D)) if want_y else None
    out = np.empty((tokens, D)) if want_out else None
    h_out = np.empty((nb, D, N)) if want_h_out else None
    t0 = time.perf_counter()
    rc = (lib or _load()).lib.ref_selective_scan(
        1 if reverse else 0, nb, off.ctypes.data_as(_i64ptr), D, N,
        _ptr(x), _ptr(dt), _ptr(Bm), _ptr(Cm), _ptr(A), _ptr(Dskip),
        1 if delta_softplus else 0, _ptr(h_in), _ptr(h_out), _ptr(y),
        _ptr(res), float(s), _ptr(out), int(nthreads))
    if timing is not None:
        timing["seconds"] = time.perf_counter() - t0
    if rc != 0:
        raise ValueError("oracle rejected its arguments (rc=%d)" % rc)
    return {"y": y, "out": out, "h_out": h_out}


RES_KINDS = {"none": 0, "x": 1, "separate": 2}


def selective_scan_backward(x, dt, Bm, Cm, A, Dskip=None, *, reverse: bool, dout,
                            dh_out=None, res_kind: str = "none", s: float = 0.0,
                            seq_offsets=None, batch=None, seqlen=None,
                            delta_softplus: bool = True, h_in=None, nthreads: int = 0,
                            timing: dict | None = None, lib: OracleLib | None = None):
    """Gradients of the scan with readout (and residual ``res_kind``: "none",
    "x" or "separate") for ``dout`` = dL/dout [tokens, D] and ``dh_out`` =
    dL/dh_out [batch, D, N] (or None). Returns fp64 arrays ``dx``, ``ddt``
    [tokens, D], ``dBm``, ``dCm`` [tokens, N], ``dA`` [D, N], ``dDskip`` [D],
    ``dh_in`` [batch, D, N] and the scalar ``ds``. A separate residual's
    gradient is dout itself and is not returned."""
    x, dt, Bm, Cm, A = _f64(x), _f64(dt), _f64(Bm), _f64(Cm), _f64(A)
    Dskip, h_in, dout, dh_out = _f64(Dskip), _f64(h_in), _f64(dout), _f64(dh_out)
    tokens, D = x.shape
    N = A.shape[1]
    off = _offsets(seq_offsets, batch, seqlen, tokens)
    nb = off.shape[0] - 1
    assert dt.shape == (tokens, D) and dout.shape == (tokens, D)
    assert Bm.shape == (tokens, N) and Cm.shape == (tokens, N) and A.shape == (D, N)
    if h_in is not None:
        h_in = h_in.reshape(nb, D, N)
    if dh_out is not None:
        dh_out = dh_out.reshape(nb, D, N)
    r = {"dx": np.empty((tokens, D)), "ddt": np.empty((tokens, D)),
         "dBm": np.empty((tokens, N)), "dCm": np.empty((tokens, N)), "dA": np.empty((D, N)),
         "dDskip": np.empty(D), "dh_in": np.empty((nb, D, N)), "ds": np.empty(1)}
    t0 = time.perf_counter()
    rc = (lib or _load()).lib.ref_selective_scan_backward(
        1 if reverse else 0, nb, off.ctypes.data_as(_i64ptr), D, N,
        _ptr(x), _ptr(dt), _ptr(Bm), _ptr(Cm), _ptr(A), _ptr(Dskip),
        1 if delta_softplus else 0, _ptr(h_in), RES_KINDS[res_kind], float(s),
        _ptr(dout), _ptr(dh_out), _ptr(r["dx"]), _ptr(r["ddt"]), _ptr(r["dBm"]),
        _ptr(r["dCm"]), _ptr(r["dA"]), _ptr(r["dDskip"]), _ptr(r["dh_in"]), _ptr(r["ds"]),
        int(nthreads))
    if timing is not None:
        timing["seconds"] = time.perf_counter() - t0
    if rc != 0:
        raise ValueError("oracle backward rejected its arguments (rc=%d)" % rc)
    r["ds"] = float(r["ds"][0])
    return r


def bidir_scan(x, dt, Bm, Cm, A, Dskip=None, *, rev=None, res=None, s: float = 0.0,
               seq_offsets=None, batch=None, seqlen=None, delta_softplus: bool = True,
               h_in=None, want_h_out=False, want_out=True, nthreads: int = 0,
               timing: dict | None = None, lib: OracleLib | None = None):
    """Bidirectional full-window scan: the forward scan (parameters dt, Bm, Cm,
    A, Dskip; from h_in) plus the reverse scan (parameters ``rev``, a dict with
    the same keys, each defaulting to the forward's; from zero) of the same x.
    Returns fp64 ``y`` = y_forward + y_reverse, ``out`` (res + s*y, s == 0:
    res; y without res) and the forward's final state ``h_out``."""
    rev = dict(rev or {})
    unknown = set(rev) - {"dt", "Bm", "Cm", "A", "Dskip"}
    if unknown:
        raise ValueError("unknown reverse parameters %s" % sorted(unknown))
    f = {"dt": _f64(dt), "Bm": _f64(Bm), "Cm": _f64(Cm), "A": _f64(A), "Dskip": _f64(Dskip)}
    r = {k: (_f64(rev[k]) if k in rev else f[k]) for k in f}
    x, h_in, res = _f64(x), _f64(h_in), _f64(res)
    tokens, D = x.shape
    N = f["A"].shape[1]
    off = _offsets(seq_offsets, batch, seqlen, tokens)
    nb = off.shape[0] - 1
    for p in (f, r):
        assert p["dt"].shape == (tokens, D) and p["A"].shape == (D, N)
        assert p["Bm"].shape == (tokens, N) and p["Cm"].shape == (tokens, N)
        assert p["Dskip"] is None or p["Dskip"].shape == (D,)
    if h_in is not None:
        h_in = h_in.reshape(nb, D, N)
    if res is not None:
        assert res.shape == (tokens, D)
    y = np.empty((tokens, D))
    out = np.empty((tokens, D)) if want_out else None
    h_out = np.empty((nb, D, N)) if want_h_out else None
    t0 = time.perf_counter()
    rc = (lib or _load()).lib.ref_bidir_scan(
        nb, off.ctypes.data_as(_i64ptr), D, N, _ptr(x),
        _ptr(f["dt"]), _ptr(f["Bm"]), _ptr(f["Cm"]), _ptr(f["A"]), _ptr(f["Dskip"]),
        _ptr(r["dt"]), _ptr(r["Bm"]), _ptr(r["Cm"]), _ptr(r["A"]), _ptr(r["Dskip"]),
        1 if delta_softplus else 0, _ptr(h_in), _ptr(h_out), _ptr(y), _ptr(res), float(s),
        _ptr(out), int(nthreads))
    if timing is not None:
        timing["seconds"] = time.perf_counter() - t0
    if rc != 0:
        raise ValueError("oracle bidirectional scan rejected its arguments (rc=%d)" % rc)
    return {"y": y, "out": out, "h_out": h_out}


def _round_to(a, store):
    """The value of fp64 array ``a`` once stored as ``store`` ("f32": IEEE
    single; "bf16": the upper 16 bits of the single after round-to-nearest-even;
    None: kept in fp64)."""
    if store is None:
        return a
    f = np.asarray(a, dtype=np.float64).astype(np.float32)
    if store == "f32":
        return f.astype(np.float64)
    u = f.view(np.uint32).astype(np.uint64)
    keep = (u >> 16) & 1                           # ties go to the even upper half
    u = ((u + 0x7FFF + keep) >> 16) << 16
    out = (u & 0xFFFFFFFF).astype(np.uint32).view(np.float32).astype(np.float64)
    return np.where(np.isnan(f), np.float64("nan"), out)


def _silu(v):
    return v / (1.0 + np.exp(-v))


def sidecar_forward(hidden, W_in, conv_w, conv_b, W_x, W_dt, dt_bias, A, Dskip, W_out, *,
                    s: float, seq_offsets=None, batch=None, seqlen=None, store=None,
                    nthreads: int = 0, timing: dict | None = None):
    """The R2L sidecar block around the reverse scan, one plain reading of a
    Mamba block run over the reversed sequence (the pages name a Mamba sidecar
    and give none of its internals):

        [x | z] = hidden W_in^T                       (d_model -> 2 d_inner)
        u_t     = SiLU(conv_b + sum_j conv_w[:, K-1-j] * x_{t+j})   (the causal
                  depthwise conv of the reversed sequence: taps look right,
                  zero past each sequence's last token)
        [r | B | C] = u W_x^T                          (d_inner -> R + 2N)
        dt      = r W_dt^T + dt_bias                   (Delta = softplus(dt) in the scan)
        y       = reverse selective scan of u (dt, B, C, A, Dskip)
        g       = y * SiLU(z)
        out     = hidden + s * g W_out^T               (s == 0: hidden itself)

    All arrays are fp64 [rows, cols] with the weights as [out, in]. ``store``
    ("bf16", "f32" or None) rounds every intermediate the GPU path stores
    (x|z, u, r|B|C, r W_dt^T, g) to that type, as the GPU does; the sums
    themselves are fp64. Returns a dict with ``out`` and the intermediates."""
    hidden, W_in, W_x, W_dt, W_out = (_f64(a) for a in (hidden, W_in, W_x, W_dt, W_out))
    conv_w, conv_b, dt_bias, A, Dskip = (_f64(a) for a in (conv_w, conv_b, dt_bias, A, Dskip))
    T, dm = hidden.shape
    di, N, K = W_dt.shape[0], A.shape[1], conv_w.shape[1]
    R = W_dt.shape[1]
    conv_b = np.zeros(di) if conv_b is None else conv_b      # absent terms are zero
    dt_bias = np.zeros(di) if dt_bias is None else dt_bias
    off = _offsets(seq_offsets, batch, seqlen, T)
    t0 = time.perf_counter()
    xz = _round_to(hidden @ W_in.T, store)
    x, z = xz[:, :di], xz[:, di:]
    pre = np.empty((T, di))
    for b in range(off.shape[0] - 1):
        for t in range(off[b], off[b + 1]):
            acc = conv_b.copy()
            for j in range(K):
                if t + j < off[b + 1]:
                    acc = acc + conv_w[:, K - 1 - j] * x[t + j]
            pre[t] = acc
    u = _round_to(_silu(pre), store)
    xdbl = _round_to(u @ W_x.T, store)
    dt = _round_to(xdbl[:, :R] @ W_dt.T, store) + dt_bias[None, :]
    Bm, Cm = xdbl[:, R:R + N], xdbl[:, R + N:R + 2 * N]
    y = selective_scan(u, dt, Bm, Cm, A, Dskip, reverse=True, seq_offsets=off,
                       nthreads=nthreads)["y"]
    g = _round_to(y * _silu(z), store)
    o = g @ W_out.T
    out = hidden.copy() if s == 0.0 else hidden + s * o
    if timing is not None:
        timing["seconds"] = time.perf_counter() - t0
    return {"out": out, "xz": xz, "u": u, "xdbl": xdbl, "dt": dt, "y": y, "g": g, "o": o}


def r2l_scan(x, dt, Bm, Cm, A, Dskip=None, *, res=None, s=0.0, **kw):
    """R2L stream: reverse scan + readout, then out = res + s*y (s == 0: res)."""
    kw.setdefault("want_out", True)
    return selective_scan(x, dt, Bm, Cm, A, Dskip, reverse=True, res=res, s=s, **kw)


def prefix_scan_state(x, dt, Bm, A, **kw):
    """Forward-only boundary state after each prefix (state only, no readout)."""
    r = selective_scan(x, dt, Bm, None, A, None, reverse=False, want_y=False,
                       want_h_out=True, **kw)
    return r["h_out"]


def block_commit_state(state, x, dt, Bm, A, **kw):
    """Cached boundary state advanced over each committed block."""
    r = selective_scan(x, dt, Bm, None, A, None, reverse=False, want_y=False,
                       want_h_out=True, h_in=state, **kw)
    return r["h_out"]
