"""GPU parity of the training pair r2l_scan_save / r2l_scan_backward_saved
(through the C ABI): the saving forward against the oracle's fp64 forward,
the backward from its checkpoints against the oracle's fp64 backward, and,
where neither plan chunks, both bit for bit against r2l_scan and
r2l_scan_backward (the same kernels and the same arithmetic).

Tolerances are those of the forward and backward parity tests: outputs
max|err| / max|ref| <= 1e-5 (fp32) or 2e-2 and one bf16 ulp per element
(bf16), states 1e-5; gradients 1e-5 (fp32) or 2e-2 and one bf16 ulp plus
1e-5 * max|ref| per element for dx and ddt stored in bf16.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import reverse_mamba_selective_amd as r2l
import synth
from gpu_util import bits, check_state, check_y, dev, dev32, gpu  # noqa: F401
from test_gpu_backward import FP32_GRADS, GRAD_TOL, check_grad

pytestmark = pytest.mark.gpu


def device_inputs(inp, dense, dtype):
    B = inp.batch

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
    return x, kw, shaped


def run_saved(inp, dense, res_kind, s, with_hin, with_dhout, seed, chunk_tokens=0, reverse=True,
              softplus=True):
    """Saving forward, then the backward from its checkpoints; both against
    the oracle (reverse False: the left-to-right pair)."""
    dtype = inp.dtype
    B, D = inp.batch, inp.x.shape[1]
    rng = np.random.default_rng(seed)
    dout_np = synth.round_bf16(rng.standard_normal(inp.x.shape)) if dtype == "bf16" else \
        rng.standard_normal(inp.x.shape).astype(np.float32)
    dh_out_np = rng.standard_normal((B, D, 16)).astype(np.float32) if with_dhout else None
    h0 = synth.initial_state(seed, B, D, 16) if with_hin else None
    res_np = {"none": None, "x": inp.x,
              "separate": synth.scan_inputs(seed + 1, inp.lengths, D=D, dtype=dtype).x}[res_kind]
    fwd = oracle.selective_scan(inp.x, inp.dt, inp.Bm, inp.Cm, inp.A, inp.Dskip, reverse=reverse,
                                seq_offsets=inp.offsets, h_in=h0, want_h_out=True, res=res_np,
                                s=s, want_out=res_np is not None, delta_softplus=softplus)
    ref = oracle.selective_scan_backward(
        inp.x, inp.dt, inp.Bm, inp.Cm, inp.A, inp.Dskip, reverse=reverse, dout=dout_np,
        dh_out=dh_out_np, res_kind=res_kind, s=s, seq_offsets=inp.offsets, h_in=h0,
        delta_softplus=softplus)

    x, kw, shaped = device_inputs(inp, dense, dtype)
    save = r2l.r2l_scan_save if reverse else r2l.prefix_scan_save
    bwd = r2l.r2l_scan_backward if reverse else r2l.prefix_scan_backward
    res = None if res_np is None else (x if res_kind == "x" else shaped(dev(res_np, dtype)))
    h_in = dev32(h0) if with_hin else None
    h_out = torch.empty((B, D, 16), dtype=torch.float32, device="cuda")
    out, ckpt = save(x, **kw, h_in=h_in, h_out=h_out, res=res, s=s, chunk_tokens=chunk_tokens,
                     delta_softplus=softplus)
    g = bwd(x, **kw, dout=shaped(dev(dout_np, dtype)),
            dh_out=dev32(dh_out_np) if with_dhout else None, h_in=h_in, res=res, s=s, ckpt=ckpt,
            delta_softplus=softplus)
    torch.cuda.synchronize()
    if res is not None and s == 0.0:
        assert np.array_equal(bits(out), bits(res)), "s == 0: out is not res bit for bit"
    else:
        check_y(out.reshape(-1, D), fwd["out"] if res is not None else fwd["y"], dtype, "out")
    check_state(h_out, fwd["h_out"], "h_out")
    for name in ("dx", "ddt") + FP32_GRADS:
        check_grad(name, g[name], ref[name], dtype)
    if res is not None:
        e = abs(g["ds"].item() - ref["ds"]) / max(abs(ref["ds"]), 1e-30)
        assert e <= GRAD_TOL, "ds: %.3e" % e
    return out, g


# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("res_kind", ["none", "x", "separate"])
def test_saved_ragged_edges(gpu, dtype, res_kind):
    """Sequences of 0, 1 and 7..130 tokens (partial and full checkpoint groups
    and tiles), a channel tail (100 channels)."""
    lengths = [5, 0, 1, 7, 8, 9, 64, 65, 130]
    inp = synth.scan_inputs(51, lengths, D=100, dtype=dtype, dt_mean=-3.0)
    for with_hin, with_dhout in ((False, False), (True, True)):
        run_saved(inp, False, res_kind, 0.0 if res_kind == "none" else 0.4, with_hin,
                  with_dhout, seed=52)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_saved_without_softplus(gpu, dtype):
    """delta_softplus off (Delta = dt, positive draws): the saving forward and
    the backward from its checkpoints, unchunked and chunked."""
    inp = synth.scan_inputs(66, [5, 0, 1, 8, 9, 64, 65], D=100, dtype=dtype, dt_mean=0.1,
                            dt_std=0.02)
    for chunk in (0, 16):
        run_saved(inp, False, "x", 0.4, True, True, seed=67, chunk_tokens=chunk, softplus=False)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("chunk", [8, 13, 40])
def test_saved_chunked_forward(gpu, dtype, chunk):
    """A chunked saving forward (13 rounds up to 16 tokens: chunks are whole
    checkpoint groups) stores the checkpoints in its readout pass, from the
    carried chunk entry states."""
    lengths = [5, 0, 1, 64, 65, 130, 300, 9]
    inp = synth.scan_inputs(53, lengths, D=100, dtype=dtype, dt_mean=-3.0)
    run_saved(inp, False, "x", 0.6, True, True, seed=54, chunk_tokens=chunk)


def test_saved_planner_chunks(gpu):
    """Long sequences and few channels: the planner chunks the saving forward."""
    inp = synth.scan_inputs(55, [3000, 1, 700], D=64, dtype="f32")
    run_saved(inp, False, "x", 0.3, True, True, seed=56)


@pytest.mark.parametrize("res_kind", ["x", "separate"])
def test_saved_gate_closed(gpu, res_kind):
    """s = 0: out is res bit for bit, and a state-only scan stores the
    checkpoints (the backward still needs the states for dh_in and ds)."""
    inp = synth.scan_inputs(57, [40, 3, 17], D=72, dtype="bf16")
    run_saved(inp, False, res_kind, 0.0, True, True, seed=58)


@pytest.mark.parametrize("reverse", [True, False], ids=["r2l", "l2r"])
def test_saved_gate_closed_out_is_x(gpu, reverse):
    """s = 0 with out = x and a separate residual: x is overwritten by the
    residual, and the checkpoints (stored by a state-only scan) and h_out are
    still the states of the x that was passed in."""
    inp = synth.scan_inputs(64, [40, 3, 17, 0, 9], D=72, dtype="bf16")
    B, D = inp.batch, 72
    res_np = synth.scan_inputs(65, inp.lengths, D=D, dtype="bf16").x
    fwd = oracle.selective_scan(inp.x, inp.dt, inp.Bm, inp.Cm, inp.A, inp.Dskip,
                                reverse=reverse, seq_offsets=inp.offsets, want_h_out=True)
    rng = np.random.default_rng(66)
    dout_np = synth.round_bf16(rng.standard_normal(inp.x.shape))
    ref = oracle.selective_scan_backward(
        inp.x, inp.dt, inp.Bm, inp.Cm, inp.A, inp.Dskip, reverse=reverse, dout=dout_np,
        res_kind="separate", s=0.0, seq_offsets=inp.offsets)
    x, kw, _ = device_inputs(inp, False, "bf16")
    x_keep = x.clone()
    res = dev(res_np, "bf16")
    h_out = torch.empty((B, D, 16), dtype=torch.float32, device="cuda")
    save = r2l.r2l_scan_save if reverse else r2l.prefix_scan_save
    bwd = r2l.r2l_scan_backward if reverse else r2l.prefix_scan_backward
    out, ckpt = save(x, **kw, h_out=h_out, res=res, s=0.0, out=x)
    g = bwd(x_keep, **kw, dout=dev(dout_np, "bf16"), res=res, s=0.0, ckpt=ckpt)
    torch.cuda.synchronize()
    assert out.data_ptr() == x.data_ptr()
    assert np.array_equal(bits(x), bits(res)), "s == 0: out is not res bit for bit"
    check_state(h_out, fwd["h_out"], "h_out")
    for name in ("dx", "ddt") + FP32_GRADS:
        check_grad(name, g[name], ref[name], "bf16")


@pytest.mark.parametrize("dense", [True, False], ids=["dense", "ragged"])
def test_saved_matches_unsaved_bitwise(gpu, dense):
    """Unchunked, the saving forward is r2l_scan bit for bit, and the backward
    from its checkpoints is r2l_scan_backward bit for bit."""
    lengths = [32] * 8 if dense else [5, 0, 1, 7, 8, 9, 64, 65, 130]
    inp = synth.scan_inputs(59, lengths, D=256, dtype="bf16", dt_mean=-3.0)
    x, kw, shaped = device_inputs(inp, dense, "bf16")
    B, D = inp.batch, 256
    rng = np.random.default_rng(60)
    dout = shaped(dev(synth.round_bf16(rng.standard_normal(inp.x.shape)), "bf16"))
    h_in = dev32(synth.initial_state(60, B, D, 16))
    dh_out = dev32(rng.standard_normal((B, D, 16)).astype(np.float32))
    hs = [torch.empty((B, D, 16), dtype=torch.float32, device="cuda") for _ in range(2)]
    base = r2l.r2l_scan(x, **kw, h_in=h_in, h_out=hs[0], res=x, s=0.3, chunk_tokens=-1,
                        state_split=1)
    out, ckpt = r2l.r2l_scan_save(x, **kw, h_in=h_in, h_out=hs[1], res=x, s=0.3,
                                  chunk_tokens=-1)
    g0 = r2l.r2l_scan_backward(x, **kw, dout=dout, dh_out=dh_out, h_in=h_in, res=x, s=0.3,
                               chunk_tokens=-1)
    g1 = r2l.r2l_scan_backward(x, **kw, dout=dout, dh_out=dh_out, h_in=h_in, res=x, s=0.3,
                               chunk_tokens=-1, ckpt=ckpt)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), bits(base))
    assert np.array_equal(bits(hs[1]), bits(hs[0]))
    for name in g0:
        assert np.array_equal(bits(g1[name]), bits(g0[name])), name


def test_saved_repeated_and_reused(gpu):
    """The checkpoints are an input of the backward: two backward calls from
    one saving forward give the same bits, and a second saving forward into
    the same buffer (other inputs, fewer tokens) replaces what the backward
    reads."""
    inp = synth.scan_inputs(61, [48, 20, 33], D=96, dtype="f32")
    small = synth.scan_inputs(62, [9, 30], D=96, dtype="f32")
    x, kw, _ = device_inputs(inp, False, "f32")
    dout = torch.randn_like(x)
    out, ckpt = r2l.r2l_scan_save(x, **kw, res=x, s=0.5)
    g0 = r2l.r2l_scan_backward(x, **kw, dout=dout, res=x, s=0.5, ckpt=ckpt)
    g1 = r2l.r2l_scan_backward(x, **kw, dout=dout, res=x, s=0.5, ckpt=ckpt)
    torch.cuda.synchronize()
    for name in g0:
        assert np.array_equal(bits(g1[name]), bits(g0[name])), name
    run = {}
    xs, kws, _ = device_inputs(small, False, "f32")
    _, ckpt2 = r2l.r2l_scan_save(xs, **kws, res=xs, s=0.5, ckpt=ckpt)
    assert ckpt2 is ckpt
    dsm = torch.randn_like(xs)
    run["saved"] = r2l.r2l_scan_backward(xs, **kws, dout=dsm, res=xs, s=0.5, ckpt=ckpt)
    ref = oracle.selective_scan_backward(small.x, small.dt, small.Bm, small.Cm, small.A,
                                         small.Dskip, reverse=True,
                                         dout=dsm.cpu().numpy(), res_kind="x", s=0.5,
                                         seq_offsets=small.offsets)
    torch.cuda.synchronize()
    for name in ("dx", "ddt") + FP32_GRADS:
        check_grad(name, run["saved"][name], ref[name], "f32")


def test_saved_rejects_bad_checkpoints(gpu):
    inp = synth.scan_inputs(63, [40, 3], D=64, dtype="f32")
    x, kw, _ = device_inputs(inp, False, "f32")
    need = r2l.checkpoint_size(x, kw["A"], cu_seqlens=kw["cu_seqlens"],
                               max_seqlen=kw["max_seqlen"])
    assert need == (43 // 8 + 2 + 1) * 64 * 16 * 4
    short = torch.empty(need // 4 - 1, dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        r2l.r2l_scan_save(x, **kw, ckpt=short)
    with pytest.raises(r2l.R2LError):
        r2l.r2l_scan_backward(x, **kw, dout=torch.randn_like(x), ckpt=short)
    # the saving forward runs one lane per channel: a split plan is refused
    # by the library's argument checks, before anything is launched
    full = torch.empty(need // 4, dtype=torch.float32, device="cuda")
    a = r2l._fill(x, kw["dt"], kw["Bm"], kw["Cm"], kw["A"], kw["Dskip"], kw["cu_seqlens"],
                  kw["max_seqlen"], None, None, None, 0.0, torch.empty_like(x), True, 0, 2)
    with pytest.raises(r2l.R2LError):
        r2l._abi.call_save(a, full.data_ptr(), need, None)


def test_saved_bound_calls(gpu):
    """bind("r2l_scan_save") and bind_backward(ckpt=...) launch the same calls
    as the functions, bit for bit, on every launch."""
    inp = synth.scan_inputs(64, [32] * 4, D=128, dtype="bf16", dt_mean=-3.0)
    x, kw, shaped = device_inputs(inp, True, "bf16")
    dout = torch.randn_like(x)
    out0, ck0 = r2l.r2l_scan_save(x, **kw, res=x, s=0.2)
    g0 = r2l.r2l_scan_backward(x, **kw, dout=dout, res=x, s=0.2, ckpt=ck0)
    out1 = torch.empty_like(x)
    sc = r2l.bind("r2l_scan_save", x=x, res=x, s=0.2, out=out1, **kw)
    bc = r2l.bind_backward(x, **kw, dout=dout, res=x, s=0.2, ckpt=sc.ckpt)
    for _ in range(2):
        sc.launch()
        bc.launch()
        torch.cuda.synchronize()
        assert np.array_equal(bits(out1), bits(out0))
        for name in g0:
            assert np.array_equal(bits(bc.grads[name]), bits(g0[name])), name


# ---- the left-to-right pair (prefix_scan_save / prefix_scan_backward_saved) --------
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("res_kind", ["none", "x", "separate"])
def test_saved_l2r_ragged_edges(gpu, dtype, res_kind):
    """The L2R stream's saving forward and backward: sequences of 0, 1 and
    7..130 tokens, a channel tail."""
    lengths = [5, 0, 1, 7, 8, 9, 64, 65, 130]
    inp = synth.scan_inputs(71, lengths, D=100, dtype=dtype, dt_mean=-3.0)
    for with_hin, with_dhout in ((False, False), (True, True)):
        run_saved(inp, False, res_kind, 0.0 if res_kind == "none" else 0.4, with_hin,
                  with_dhout, seed=72, reverse=False)


@pytest.mark.parametrize("chunk", [13, 40])
def test_saved_l2r_chunked_forward(gpu, chunk):
    lengths = [5, 0, 1, 64, 65, 130, 300, 9]
    inp = synth.scan_inputs(73, lengths, D=100, dtype="bf16", dt_mean=-3.0)
    run_saved(inp, False, "x", 0.6, True, True, seed=74, chunk_tokens=chunk, reverse=False)


def test_saved_l2r_gate_closed(gpu):
    inp = synth.scan_inputs(75, [40, 3, 17], D=72, dtype="f32")
    run_saved(inp, False, "x", 0.0, True, True, seed=76, reverse=False)


def test_saved_l2r_matches_unsaved_bitwise(gpu):
    """Unchunked, prefix_scan_save is prefix_scan_state with readout bit for
    bit, and the backward from its checkpoints is prefix_scan_backward."""
    inp = synth.scan_inputs(77, [32] * 8, D=256, dtype="bf16", dt_mean=-3.0)
    x, kw, shaped = device_inputs(inp, True, "bf16")
    B, D = inp.batch, 256
    rng = np.random.default_rng(78)
    dout = shaped(dev(synth.round_bf16(rng.standard_normal(inp.x.shape)), "bf16"))
    h_in = dev32(synth.initial_state(78, B, D, 16))
    hs = [torch.empty((B, D, 16), dtype=torch.float32, device="cuda") for _ in range(2)]
    base = torch.empty_like(x)
    r2l.prefix_scan_state(x, kw["dt"], kw["Bm"], kw["A"], Cm=kw["Cm"], Dskip=kw["Dskip"],
                          h_in=h_in, h_out=hs[0], res=x, s=0.3, out=base, chunk_tokens=-1,
                          state_split=1)
    out, ckpt = r2l.prefix_scan_save(x, **kw, h_in=h_in, h_out=hs[1], res=x, s=0.3,
                                     chunk_tokens=-1)
    g0 = r2l.prefix_scan_backward(x, **kw, dout=dout, h_in=h_in, res=x, s=0.3, chunk_tokens=-1)
    g1 = r2l.prefix_scan_backward(x, **kw, dout=dout, h_in=h_in, res=x, s=0.3, chunk_tokens=-1,
                                  ckpt=ckpt)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), bits(base))
    assert np.array_equal(bits(hs[1]), bits(hs[0]))
    for name in g0:
        assert np.array_equal(bits(g1[name]), bits(g0[name])), name


def test_autograd_saves_only_when_needed(gpu):
    """R2LScan runs r2l_scan when no input needs a gradient and the saving
    forward otherwise (bit for bit those calls)."""
    inp = synth.scan_inputs(79, [32] * 4, D=128, dtype="f32")
    x, kw, _ = device_inputs(inp, True, "f32")
    ref0 = r2l.r2l_scan(x, **kw, res=x, s=0.25)
    ref1, _ = r2l.r2l_scan_save(x, **kw, res=x, s=0.25)
    with torch.no_grad():
        out0 = r2l.R2LScan.apply(x, kw["dt"], kw["Bm"], kw["Cm"], kw["A"], kw["Dskip"], 0.25)
    xg = x.clone().requires_grad_()
    out1 = r2l.R2LScan.apply(xg, kw["dt"], kw["Bm"], kw["Cm"], kw["A"], kw["Dskip"], 0.25)
    out1.sum().backward()
    torch.cuda.synchronize()
    assert np.array_equal(bits(out0), bits(ref0))
    assert np.array_equal(bits(out1.detach()), bits(ref1))
    assert xg.grad is not None and torch.isfinite(xg.grad).all()


def test_saved_l2r_bound_calls(gpu):
    """bind("prefix_scan_save") and bind_backward(ckpt=..., _reverse=False)
    launch the same calls as prefix_scan_save / prefix_scan_backward."""
    inp = synth.scan_inputs(80, [32] * 4, D=128, dtype="bf16", dt_mean=-3.0)
    x, kw, _ = device_inputs(inp, True, "bf16")
    dout = torch.randn_like(x)
    out0, ck0 = r2l.prefix_scan_save(x, **kw, res=x, s=0.2)
    g0 = r2l.prefix_scan_backward(x, **kw, dout=dout, res=x, s=0.2, ckpt=ck0)
    out1 = torch.empty_like(x)
    sc = r2l.bind("prefix_scan_save", x=x, res=x, s=0.2, out=out1, **kw)
    bc = r2l.bind_backward(x, **kw, dout=dout, res=x, s=0.2, ckpt=sc.ckpt, _reverse=False)
    assert bc.func == "prefix_scan_backward_saved"
    for _ in range(2):
        sc.launch()
        bc.launch()
        torch.cuda.synchronize()
        assert np.array_equal(bits(out1), bits(out0))
        for name in g0:
            assert np.array_equal(bits(bc.grads[name]), bits(g0[name])), name
