"""GPU parity of bidir_scan (through the C ABI) against the oracle's fp64
bidirectional scan on the same seeded inputs.

The tolerances are those of the single-direction scans (gpu_util): fp32
max|err| / max|ref| <= 1e-5 on y, out and the forward state; bf16 2e-2 on y
and every output element within one bf16 ulp plus the fp32 bound; s == 0
gives the residual bit for bit.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import reverse_mamba_selective_amd as r2l
import synth
from gpu_util import bits, check_state, check_y, dev, dev32, gpu, host  # noqa: F401

pytestmark = pytest.mark.gpu


def on_gpu(inp, rev, dense):
    g = {"x": dev(inp.x, inp.dtype), "dt": dev(inp.dt, inp.dtype), "Bm": dev(inp.Bm, inp.dtype),
         "Cm": dev(inp.Cm, inp.dtype), "A": dev32(inp.A), "Dskip": dev32(inp.Dskip)}
    r = None
    if rev is not None:
        r = {k: (dev32(v) if k in ("A", "Dskip") else dev(v, inp.dtype)) for k, v in rev.items()}
    kw = {}
    if dense:
        L = int(inp.lengths[0]) if inp.batch else 0
        shape = lambda t: t.view(inp.batch, L, -1)
        for k in ("x", "dt", "Bm", "Cm"):
            g[k] = shape(g[k])
        if r is not None:
            r = {k: (shape(v) if k in ("dt", "Bm", "Cm") else v) for k, v in r.items()}
    else:
        kw = dict(cu_seqlens=torch.from_numpy(inp.offsets.astype(np.int32)).cuda(),
                  max_seqlen=int(inp.lengths.max()) if inp.batch else 0)
    return g, r, kw


def run_case(inp, rev, *, dense, res_kind="none", s=0.0, with_hin=False, with_hout=False,
             seed=0, chunk_tokens=0, in_place=False):
    """bidir_scan on the GPU and the oracle; returns (out, h_out, reference)."""
    B, D = inp.batch, inp.x.shape[1]
    h0 = synth.initial_state(seed, B, D, 16) if with_hin else None
    res_np = {"none": None, "x": inp.x,
              "separate": synth.scan_inputs(seed + 1, inp.lengths, D=D, dtype=inp.dtype).x}[res_kind]
    ref = oracle.bidir_scan(inp.x, inp.dt, inp.Bm, inp.Cm, inp.A, inp.Dskip, rev=rev,
                            seq_offsets=inp.offsets, res=res_np, s=s, h_in=h0,
                            want_h_out=with_hout)
    g, r, kw = on_gpu(inp, rev, dense)
    x = g["x"].clone() if in_place else g["x"]
    res = None if res_np is None else (x if res_kind == "x" else
                                       dev(res_np, inp.dtype).view(x.shape))
    h_out = torch.empty((B, D, 16), device="cuda") if with_hout else None
    out = r2l.bidir_scan(x, g["dt"], g["Bm"], g["Cm"], g["A"], g["Dskip"], rev=r, res=res, s=s,
                         h_in=dev32(h0) if with_hin else None, h_out=h_out,
                         out=x if in_place else None, chunk_tokens=chunk_tokens, **kw)
    torch.cuda.synchronize()
    return out, h_out, ref, res


def check_case(inp, rev, what="", **kw):
    out, h_out, ref, res = run_case(inp, rev, **kw)
    D = inp.x.shape[1]
    got = out.reshape(-1, D)
    if kw.get("res_kind", "none") == "none":
        check_y(got, ref["y"], inp.dtype, what + " y")
    elif kw.get("s", 0.0) == 0.0:
        assert np.array_equal(bits(got), bits(res.reshape(-1, D))), what + " s = 0"
    else:
        check_y(got, ref["out"], inp.dtype, what + " out")
    if kw.get("with_hout"):
        check_state(h_out, ref["h_out"], what + " forward state")
    return out


# ---------------------------------------------------------------------------
@pytest.mark.parametrize("shared", [True, False], ids=["shared", "separate"])
def test_bidir_tiny_fp32(gpu, shared):
    inp = synth.tiny_inputs()
    rev = None if shared else synth.reverse_params(7, inp.lengths, 64)
    check_case(inp, rev, dense=True, with_hin=True, with_hout=True, seed=41)
    check_case(inp, rev, dense=True, res_kind="x", s=0.5, seed=41)


@pytest.mark.parametrize("rev_kind", ["shared", "separate", "partial"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("res_kind,s", [("none", 0.0), ("x", 0.3), ("separate", -0.6)])
def test_bidir_ragged_edges(gpu, dtype, res_kind, s, rev_kind):
    """Sequences of 0, 1 and 7..130 tokens (tile and prefetch-group tails), 100
    channels (a tile tail); each direction's parameters shared, separate, or
    only dt and A of the reverse direction its own."""
    lengths = [5, 0, 1, 7, 8, 9, 64, 65, 130]
    inp = synth.scan_inputs(42, lengths, D=100, dtype=dtype)
    rev = {"shared": None,
           "separate": synth.reverse_params(42, lengths, 100, dtype=dtype),
           "partial": {k: v for k, v in synth.reverse_params(42, lengths, 100, dtype=dtype).items()
                       if k in ("dt", "A")}}[rev_kind]
    check_case(inp, rev, dense=False, res_kind=res_kind, s=s, with_hin=True, with_hout=True,
               seed=43)


@pytest.mark.parametrize("rev_kind", ["shared", "separate"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("res_kind,s", [("none", 0.0), ("x", 0.3), ("separate", -0.6)])
def test_bidir_short_windows(gpu, dtype, res_kind, s, rev_kind):
    """Windows of at most 32 tokens, whose reverse readout stays in LDS: lengths
    0, 1 and 5..32 (prefetch-group tails and a full 32), a channel tile tail."""
    lengths = [5, 0, 1, 7, 8, 9, 31, 32, 16]
    inp = synth.scan_inputs(52, lengths, D=100, dtype=dtype)
    rev = None if rev_kind == "shared" else synth.reverse_params(52, lengths, 100, dtype=dtype)
    check_case(inp, rev, dense=False, res_kind=res_kind, s=s, with_hin=True, with_hout=True,
               seed=53)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bidir_chunked_plans(gpu, dtype):
    """Chunked plans (the reverse direction's plan writing the fp32 rows, then
    the forward one adding them) on long-memory inputs, where dropping a carry
    would be far outside the tolerance; against the oracle and the fused plan."""
    lengths = [700, 1, 0, 333, 64, 1025]
    inp = synth.scan_inputs(44, lengths, D=96, dtype=dtype, dt_mean=-6.0)
    rev = synth.reverse_params(44, lengths, 96, dtype=dtype, dt_mean=-6.0)
    for chunk in (100, 32):
        check_case(inp, rev, what="chunk %d" % chunk, dense=False, res_kind="x", s=0.7,
                   with_hin=True, with_hout=True, seed=45, chunk_tokens=chunk)
    check_case(inp, rev, what="chunk 100 y", dense=False, seed=45, chunk_tokens=100)


def test_bidir_long_window_default_plan(gpu):
    """A full window long enough for the default plan to chunk (2 x 4096 tokens,
    512 channels, bf16, out = y)."""
    inp = synth.scan_inputs(46, [4096] * 2, D=512, dtype="bf16")
    rev = synth.reverse_params(46, [4096] * 2, 512, dtype="bf16")
    g, _, _ = on_gpu(inp, None, True)
    plan = r2l.bind("bidir_scan", x=g["x"], dt=g["dt"], Bm=g["Bm"], Cm=g["Cm"], A=g["A"],
                    out=torch.empty_like(g["x"])).plan()
    assert plan["chunked"] == 1 and plan["launches"] == 6
    check_case(inp, rev, dense=True, with_hout=True, seed=47)


def test_bidir_gate_zero(gpu):
    """s = 0: out is the residual bit for bit (no readout), the forward state is
    still produced; in place (out = x = res) nothing changes."""
    inp = synth.scan_inputs(48, [40, 3, 0, 17], D=72, dtype="bf16")
    rev = synth.reverse_params(48, inp.lengths, 72, dtype="bf16")
    for res_kind in ("x", "separate"):
        check_case(inp, rev, dense=False, res_kind=res_kind, s=0.0, with_hin=True,
                   with_hout=True, seed=49)
    before = dev(inp.x, "bf16")
    out, _, _, _ = run_case(inp, rev, dense=False, res_kind="x", s=0.0, in_place=True, seed=49)
    assert np.array_equal(bits(out), bits(before))


def test_bidir_in_place_hook_bf16(gpu):
    """The denoising-window shape (64 x 32 x 2048, bf16) in place: out = x = res."""
    inp = synth.bidir_inputs()
    rev = synth.bidir_reverse()
    check_case(inp, rev, dense=True, res_kind="x", s=float(synth.bidir_gates()[0]),
               in_place=True, seed=50)


def test_bidir_window_bf16_y(gpu):
    inp = synth.bidir_inputs(6)
    rev = synth.bidir_reverse(6)
    check_case(inp, rev, dense=True, with_hout=True, seed=51)


@pytest.mark.parametrize("lengths", [[9, 0, 1, 70, 33], [9, 0, 1, 32, 20]],
                         ids=["workspace_rows", "lds_rows"])
def test_bidir_direction_sums_exact(gpu, lengths):
    """A = 0, Delta = 1, one unit state, integer x: y_t is the prefix sum plus
    twice the suffix sum of the sequence, exactly (fp32, |sums| < 2^24); with
    the reverse readout in the workspace (a 70-token window) and in LDS (at
    most 32 tokens)."""
    inp = synth.scan_inputs(52, lengths, D=40, dtype="f32")
    r = np.random.default_rng(53)
    x = r.integers(-8, 9, inp.x.shape).astype(np.float32)
    T = x.shape[0]
    unit = np.zeros((T, 16), np.float32)
    unit[:, 0] = 1.0
    dt1 = np.ones_like(x)
    A0 = np.zeros((40, 16), np.float32)
    cu = torch.from_numpy(inp.offsets.astype(np.int32)).cuda()
    y = r2l.bidir_scan(dev32(x), dev32(dt1), dev32(unit), dev32(unit), dev32(A0),
                       rev={"Bm": dev32(2 * unit)}, cu_seqlens=cu, delta_softplus=False)
    got = host(y)
    for b in range(len(lengths)):
        sl = slice(inp.offsets[b], inp.offsets[b + 1])
        xs = x[sl].astype(np.float64)
        expect = np.cumsum(xs, axis=0) + 2.0 * np.cumsum(xs[::-1], axis=0)[::-1]
        assert np.array_equal(got[sl], expect), b


def test_bidir_is_deterministic_and_plans_agree(gpu):
    inp = synth.scan_inputs(54, [300, 129, 64], D=160, dtype="f32")
    rev = synth.reverse_params(54, inp.lengths, 160)
    g, r, kw = on_gpu(inp, rev, False)
    args = (g["x"], g["dt"], g["Bm"], g["Cm"], g["A"], g["Dskip"])
    a = r2l.bidir_scan(*args, rev=r, **kw)
    b = r2l.bidir_scan(*args, rev=r, **kw)
    assert np.array_equal(bits(a), bits(b))
    c = r2l.bidir_scan(*args, rev=r, chunk_tokens=64, **kw)
    ref = oracle.bidir_scan(inp.x, inp.dt, inp.Bm, inp.Cm, inp.A, inp.Dskip, rev=rev,
                            seq_offsets=inp.offsets)
    check_y(c, ref["y"], "f32", "chunked")
    check_y(a, ref["y"], "f32", "fused")
    torch.cuda.synchronize()


def test_bidir_empty(gpu):
    A = torch.full((32, 16), -1.0, device="cuda")
    x = torch.zeros((0, 32), device="cuda")
    e16 = torch.zeros((0, 16), device="cuda")
    cu = torch.zeros(4, dtype=torch.int32, device="cuda")
    h0 = torch.randn((3, 32, 16), device="cuda")
    h1 = torch.empty_like(h0)
    out = r2l.bidir_scan(x, x, e16, e16, A, cu_seqlens=cu, max_seqlen=0, h_in=h0, h_out=h1)
    torch.cuda.synchronize()
    assert out.shape == (0, 32) and torch.equal(h1, h0)
