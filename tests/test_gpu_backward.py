"""GPU parity of r2l_scan_backward (through the C ABI) against the oracle's
fp64 backward on the same seeded inputs.

Tolerances: fp32 gradients (dBm, dCm, dA, dDskip, dh_in, ds, and dx / ddt for
fp32 inputs) max|err| / max|ref| <= 1e-5, the fp32 bar of the forward: fp32
arithmetic whose sums run over up to a few thousand terms (tokens x sequences
for dA, channels for dBm and dCm) in a fixed order; measured errors stay below
1e-6. dx and ddt for bf16 inputs (stored in bf16): max|err| / max|ref| <= 2e-2
and every element within one bf16 ulp of the oracle's value plus
1e-5 * max|ref| (computed in fp32, rounded once).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import reverse_mamba_selective_amd as r2l
import synth
from gpu_util import bf16_ulp, bits, dev, dev32, gpu, host, report  # noqa: F401

pytestmark = pytest.mark.gpu

GRAD_TOL = 1e-5
FP32_GRADS = ("dBm", "dCm", "dA", "dDskip", "dh_in")


def rel(got, ref):
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64).reshape(ref.shape)
    if ref.size == 0:
        return 0.0
    return float(np.max(np.abs(got - ref)) / max(float(np.max(np.abs(ref))), 1e-30))


def check_grad(name, got_t, ref, dtype):
    got = host(got_t).reshape(np.shape(ref))
    e = rel(got, ref)
    rounded = dtype == "bf16" and name in ("dx", "ddt")   # stored as bf16
    tol = 2e-2 if rounded else GRAD_TOL
    report("grad " + name, e, tol)
    assert e <= tol, "%s: max|err|/max|ref| = %.3e" % (name, e)
    if rounded and np.size(ref):
        ref = np.asarray(ref, dtype=np.float64)
        slack = bf16_ulp(ref) + GRAD_TOL * np.max(np.abs(ref))
        worst = float(np.max(np.abs(got - ref) / slack))
        assert worst <= 1.0, "%s: an element is %.2f x (1 bf16 ulp + bound) off" % (name, worst)


def run_case(inp, dense, res_kind, s, with_hin, with_dhout, seed, dtype=None, reverse=True,
             chunk_tokens=0, softplus=True):
    dtype = dtype or inp.dtype
    B, D = inp.batch, inp.x.shape[1]
    rng = np.random.default_rng(seed)
    dout_np = synth.round_bf16(rng.standard_normal(inp.x.shape)) if dtype == "bf16" else \
        rng.standard_normal(inp.x.shape).astype(np.float32)
    dh_out_np = rng.standard_normal((B, D, 16)).astype(np.float32) if with_dhout else None
    h0 = synth.initial_state(seed, B, D, 16) if with_hin else None
    res_np = {"none": None, "x": inp.x,
              "separate": synth.scan_inputs(seed + 1, inp.lengths, D=D, dtype=dtype).x}[res_kind]
    ref = oracle.selective_scan_backward(
        inp.x, inp.dt, inp.Bm, inp.Cm, inp.A, inp.Dskip, reverse=reverse, dout=dout_np,
        dh_out=dh_out_np, res_kind=res_kind, s=s, seq_offsets=inp.offsets, h_in=h0,
        delta_softplus=softplus)

    def shaped(t):
        if dense:
            L = int(inp.lengths[0]) if B else 0
            return t.view(B, L, -1)
        return t

    x = shaped(dev(inp.x, dtype))
    kw = dict(dt=shaped(dev(inp.dt, dtype)), Bm=shaped(dev(inp.Bm, dtype)),
              Cm=shaped(dev(inp.Cm, dtype)), A=dev32(inp.A), Dskip=dev32(inp.Dskip))
    if not dense:
        kw.update(cu_seqlens=torch.from_numpy(inp.offsets.astype(np.int32)).cuda(),
                  max_seqlen=int(inp.lengths.max()) if B else 0)
    res = None if res_np is None else (x if res_kind == "x" else shaped(dev(res_np, dtype)))
    bwd = r2l.r2l_scan_backward if reverse else r2l.prefix_scan_backward
    g = bwd(x, **kw, dout=shaped(dev(dout_np, dtype)),
                              dh_out=dev32(dh_out_np) if with_dhout else None,
                              h_in=dev32(h0) if with_hin else None, res=res, s=s,
                              chunk_tokens=chunk_tokens, delta_softplus=softplus)
    torch.cuda.synchronize()
    for name in ("dx", "ddt") + FP32_GRADS:
        check_grad(name, g[name], ref[name], dtype)
    if res is not None:
        e = abs(g["ds"].item() - ref["ds"]) / max(abs(ref["ds"]), 1e-30)
        report("grad ds", e, GRAD_TOL)
        assert e <= GRAD_TOL, "ds: %.3e" % e
    return g


# ---------------------------------------------------------------------------
@pytest.mark.parametrize("res_kind,s", [("none", 0.0), ("x", 0.5), ("separate", -0.7)])
def test_backward_tiny_fp32(gpu, res_kind, s):
    inp = synth.tiny_inputs()
    run_case(inp, True, res_kind, s, with_hin=True, with_dhout=True, seed=31)


@pytest.mark.parametrize("reverse", [True, False], ids=["r2l", "forward"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("res_kind", ["none", "x", "separate"])
def test_backward_ragged_edges(gpu, dtype, res_kind, reverse):
    """Sequences of 0, 1 and 7..130 tokens (partial and full checkpoint groups
    and tiles), a channel tail (100 channels: one full tile of 64 and 36)."""
    lengths = [5, 0, 1, 7, 8, 9, 64, 65, 130]
    inp = synth.scan_inputs(32, lengths, D=100, dtype=dtype, dt_mean=-3.0)
    for with_hin, with_dhout in ((False, False), (True, True)):
        run_case(inp, False, res_kind, 0.0 if res_kind == "none" else 0.4, with_hin, with_dhout,
                 seed=33, reverse=reverse)


@pytest.mark.parametrize("reverse", [True, False], ids=["r2l", "forward"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("chunk", [8, 13, 40])
def test_backward_chunked_state_pass(gpu, dtype, chunk, reverse):
    """The forward state pass cut into chunks scanned from zero (13 rounds up
    to 16 tokens: chunks are whole checkpoint groups), the carry of the chunk
    entry states and phase 2's fix-up of the chunk-local checkpoints; sequences
    of 0 to 300 tokens, h_in and dh_out given."""
    lengths = [5, 0, 1, 64, 65, 130, 300, 9]
    inp = synth.scan_inputs(41, lengths, D=100, dtype=dtype, dt_mean=-3.0)
    for res_kind, with_hin in (("x", True), ("none", False)):
        run_case(inp, False, res_kind, 0.0 if res_kind == "none" else 0.6, with_hin, True,
                 seed=42, reverse=reverse, chunk_tokens=chunk)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_without_softplus(gpu, dtype):
    """delta_softplus off: Delta is dt itself (positive draws). The backward
    kernel's instantiation without softplus reads dt on every lane of a
    channel for every token, the softplus one on one lane per token."""
    lengths = [5, 0, 1, 8, 9, 64, 65]
    inp = synth.scan_inputs(49, lengths, D=100, dtype=dtype, dt_mean=0.1, dt_std=0.02)
    for res_kind in ("none", "x"):
        run_case(inp, False, res_kind, 0.0 if res_kind == "none" else 0.4, with_hin=True,
                 with_dhout=True, seed=50, softplus=False)


def test_backward_long_few_channels(gpu):
    """Long sequences and few channels: the planner chunks the state pass
    (3000 tokens, 64 channels: 256-token chunks)."""
    inp = synth.scan_inputs(43, [3000, 1, 700], D=64, dtype="f32")
    run_case(inp, False, "x", 0.3, with_hin=True, with_dhout=True, seed=44)


def test_backward_gate_zero(gpu):
    """s = 0: dL/dy = 0, so only ds (and dx = dout when res is x) survive."""
    inp = synth.scan_inputs(34, [40, 3], D=72, dtype="f32")
    g = run_case(inp, False, "x", 0.0, with_hin=True, with_dhout=False, seed=35)
    assert not g["dBm"].any() and not g["dA"].any()


def test_backward_denoise_hook_bf16(gpu):
    """The denoising hook at full size (64 x 32 x 2048, res = x, s from the gates)."""
    s = float(synth.denoise_gates()[2])
    inp = synth.denoise_hook_inputs(2)
    run_case(inp, True, "x", s, with_hin=False, with_dhout=False, seed=36)


def test_backward_l2r_ablation_hook_bf16(gpu):
    """prefix_scan_backward at the denoising hook's full size (the L2R ablation)."""
    s = float(synth.denoise_gates()[4])
    inp = synth.denoise_hook_inputs(4)
    run_case(inp, True, "x", s, with_hin=False, with_dhout=True, seed=40, reverse=False)


def test_backward_is_deterministic(gpu):
    inp = synth.scan_inputs(37, [90, 33, 64], D=160, dtype="bf16")
    x = dev(inp.x, "bf16")
    kw = dict(dt=dev(inp.dt, "bf16"), Bm=dev(inp.Bm, "bf16"), Cm=dev(inp.Cm, "bf16"),
              A=dev32(inp.A), Dskip=dev32(inp.Dskip),
              cu_seqlens=torch.from_numpy(inp.offsets.astype(np.int32)).cuda(), max_seqlen=90,
              dout=torch.randn_like(x), res=x, s=0.3)
    for chunk in (0, 16):   # whole and chunked state pass
        a = r2l.r2l_scan_backward(x, **kw, chunk_tokens=chunk)
        for _ in range(2):
            b = r2l.r2l_scan_backward(x, **kw, chunk_tokens=chunk)
            for k in a:
                assert np.array_equal(bits(a[k]), bits(b[k])), k
    torch.cuda.synchronize()


def test_backward_empty(gpu):
    A = torch.full((32, 16), -1.0, device="cuda")
    x = torch.zeros((0, 32), device="cuda")
    e16 = torch.zeros((0, 16), device="cuda")
    cu = torch.zeros(4, dtype=torch.int32, device="cuda")
    dh = torch.randn((3, 32, 16), device="cuda")
    g = r2l.r2l_scan_backward(x, x, e16, e16, A, torch.ones(32, device="cuda"), dout=x,
                              cu_seqlens=cu, max_seqlen=0, dh_out=dh, res=x, s=0.5)
    assert torch.equal(g["dh_in"], dh)
    assert not g["dA"].any() and not g["dDskip"].any() and g["ds"].item() == 0.0
    torch.cuda.synchronize()


@pytest.mark.parametrize("s0", [0.0, 0.3])
@pytest.mark.parametrize("saved", [True, False], ids=["saved", "unsaved"])
def test_autograd_learnable_gate(gpu, s0, saved):
    """s as a learnable one-element tensor (initialised at zero, as on the pages)
    gets ds = sum(dout * y) from the oracle's backward, through the saving
    forward's checkpoints (x needs a gradient too) or the backward's own state
    pass (s alone); at s = 0 every other gradient but dx = dout is zero."""
    inp = synth.scan_inputs(40, [40] * 3, D=80, dtype="f32")
    rng = np.random.default_rng(41)
    dout = rng.standard_normal(inp.x.shape)
    ref = oracle.selective_scan_backward(inp.x, inp.dt, inp.Bm, inp.Cm, inp.A, inp.Dskip,
                                         reverse=True, dout=dout, res_kind="x", s=s0,
                                         seq_offsets=inp.offsets)
    x = dev(inp.x, "f32").view(3, 40, -1).requires_grad_(saved)
    kw = [dev(getattr(inp, k), "f32").view(3, 40, -1) for k in ("dt", "Bm", "Cm")]
    s = torch.full((1,), s0, dtype=torch.float32, device="cuda", requires_grad=True)
    out = r2l.R2LScan.apply(x, *kw, dev32(inp.A), dev32(inp.Dskip), s)
    (out * dev32(dout).view(3, 40, -1)).sum().backward()
    torch.cuda.synchronize()
    assert s.grad is not None and s.grad.shape == s.shape
    e = abs(s.grad.item() - ref["ds"]) / max(abs(ref["ds"]), 1e-30)
    report("grad ds (autograd)", e, GRAD_TOL)
    assert e <= GRAD_TOL, "ds: %.3e" % e
    if saved:
        check_grad("dx", x.grad, ref["dx"], "f32")
        if s0 == 0.0:
            assert np.array_equal(host(x.grad).reshape(-1), dout.astype(np.float32).reshape(-1))


def test_autograd_function(gpu):
    """R2LScan.apply under torch.autograd gives the oracle's gradients."""
    inp = synth.scan_inputs(38, [48] * 3, D=96, dtype="f32")
    rng = np.random.default_rng(39)
    dout = rng.standard_normal(inp.x.shape)
    ref = oracle.selective_scan_backward(inp.x, inp.dt, inp.Bm, inp.Cm, inp.A, inp.Dskip,
                                         reverse=True, dout=dout, res_kind="x", s=0.25,
                                         seq_offsets=inp.offsets)
    t = {k: dev(getattr(inp, k), "f32").view(3, 48, -1).requires_grad_()
         for k in ("x", "dt", "Bm", "Cm")}
    A = dev32(inp.A).requires_grad_()
    Ds = dev32(inp.Dskip).requires_grad_()
    out = r2l.R2LScan.apply(t["x"], t["dt"], t["Bm"], t["Cm"], A, Ds, 0.25)
    (out * dev32(dout).view(3, 48, -1)).sum().backward()
    for name, grad in (("dx", t["x"].grad), ("ddt", t["dt"].grad), ("dBm", t["Bm"].grad),
                       ("dCm", t["Cm"].grad), ("dA", A.grad), ("dDskip", Ds.grad)):
        assert rel(host(grad).reshape(np.shape(ref[name])), ref[name]) <= GRAD_TOL, name
    torch.cuda.synchronize()
