"""GPU parity: the gfx950 kernels, called through the C ABI, against the fp64
oracle on the same seeded inputs.

Workloads (sizes as the benchmark runs them):
* tiny reverse scan, fp32, 1 x 64 tokens x 64 channels, res = x, s = 0.5
* block-restricted, fp32, 8 x (512-token prefix -> boundary state [256, 16], then
  one 32-token block): prefix state, block reverse scan, block commit, and the
  chunked-resume == full-sequence invariants
* R2LM denoising hook, bf16, 64 x 32 x 2048, res = x, s ~ U(0, 0.1)
* prefill reverse scan, bf16, 8 x 4096 x 4096 (the oracle checks sampled sequences)
* ragged serving, bf16, 256 blocks of U{16..64} x 4096: reverse scan and block
  commit (oracle on sampled sequences), and the chunked prefix-state prefill
  over prefixes of U{256..8192} tokens (a subset of the 256 prefixes)
plus the bit-exact classes and the edge cases (empty and ragged inputs, tails
of channel tiles and chunks, strides, in-place updates, every plan).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import reverse_mamba_selective_amd as r2l
import synth
from gpu_util import (STATE_TOL, TOL, bits, check_state, check_y, dev, dev32, gpu,  # noqa: F401
                      host, rel_err)

pytestmark = pytest.mark.gpu


def oracle_scan(inp, reverse=True, res=None, s=0.0, h_in=None, want_h_out=False, want_out=False,
                delta_softplus=True):
    return oracle.selective_scan(inp.x, inp.dt, inp.Bm, inp.Cm, inp.A, inp.Dskip, reverse=reverse,
                                 seq_offsets=inp.offsets, res=res, s=s, h_in=h_in,
                                 want_h_out=want_h_out, want_out=want_out,
                                 delta_softplus=delta_softplus)


def on_gpu(inp, dense=True):
    """Device tensors of a ScanInputs; dense ones as [batch, L, .] views."""
    g = {"x": dev(inp.x, inp.dtype), "dt": dev(inp.dt, inp.dtype), "Bm": dev(inp.Bm, inp.dtype),
         "Cm": dev(inp.Cm, inp.dtype), "A": dev32(inp.A), "Dskip": dev32(inp.Dskip)}
    if dense:
        L = int(inp.lengths[0]) if inp.batch else 0
        assert np.all(inp.lengths == L)
        for k in ("x", "dt", "Bm", "Cm"):
            g[k] = g[k].view(inp.batch, L, -1)
    else:
        g["cu_seqlens"] = torch.from_numpy(inp.offsets.astype(np.int32)).to("cuda")
        g["max_seqlen"] = int(inp.lengths.max()) if inp.batch else 0
    return g


def scan_kw(g):
    kw = dict(x=g["x"], dt=g["dt"], Bm=g["Bm"], Cm=g["Cm"], A=g["A"], Dskip=g["Dskip"])
    if "cu_seqlens" in g:
        kw.update(cu_seqlens=g["cu_seqlens"], max_seqlen=g["max_seqlen"])
    return kw


def flat(t):
    return t.reshape(-1, t.shape[-1])


# ---------------------------------------------------------------------------
# tiny reverse scan (fp32)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("split", [0, 1, 2, 4])
def test_tiny_r2l_fp32(gpu, split):
    inp = synth.tiny_inputs()
    ref = oracle_scan(inp, res=inp.x, s=0.5, want_out=True, want_h_out=True)
    g = on_gpu(inp)
    h_out = torch.empty((1, 64, 16), device="cuda")
    y = r2l.r2l_scan(**scan_kw(g), state_split=split, h_out=h_out)
    check_y(flat(y), ref["y"], "f32")
    check_state(h_out, ref["h_out"])
    out = r2l.r2l_scan(**scan_kw(g), res=g["x"], s=0.5, state_split=split)
    assert rel_err(host(flat(out)), ref["out"]) <= TOL["f32"]
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# block-restricted workload (fp32): prefix state, block scans, resume invariants
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("chunk", [0, -1, 96])
def test_block_restricted_fp32(gpu, chunk):
    pre, blk = synth.block_inputs()
    gp, gb = on_gpu(pre), on_gpu(blk)
    h_pre_ref = oracle.prefix_scan_state(pre.x, pre.dt, pre.Bm, pre.A, seq_offsets=pre.offsets)
    h_pre = r2l.prefix_scan_state(gp["x"], gp["dt"], gp["Bm"], gp["A"], chunk_tokens=chunk)
    check_state(h_pre, h_pre_ref, "prefix state")

    # reverse scan restricted to the active block, residual onto the hidden states
    ref_blk = oracle_scan(blk, res=blk.x, s=0.5, want_out=True)
    out = r2l.r2l_scan(**scan_kw(gb), res=gb["x"], s=0.5)
    assert rel_err(host(flat(out)), ref_blk["out"]) <= TOL["f32"]

    # the block's reverse scan equals the full reverse scan restricted to the tail
    full = synth.ScanInputs("f32", pre.lengths + blk.lengths, synth.offsets(pre.lengths + 32),
                            np.concatenate([pre.x.reshape(8, 512, -1), blk.x.reshape(8, 32, -1)],
                                           1).reshape(-1, 256),
                            np.concatenate([pre.dt.reshape(8, 512, -1), blk.dt.reshape(8, 32, -1)],
                                           1).reshape(-1, 256),
                            np.concatenate([pre.Bm.reshape(8, 512, -1), blk.Bm.reshape(8, 32, -1)],
                                           1).reshape(-1, 16),
                            np.concatenate([pre.Cm.reshape(8, 512, -1), blk.Cm.reshape(8, 32, -1)],
                                           1).reshape(-1, 16), pre.A, pre.Dskip)
    gf = on_gpu(full)
    y_full = r2l.r2l_scan(**{**scan_kw(gf), "Dskip": gp["Dskip"]}, chunk_tokens=-1)
    y_blk = r2l.r2l_scan(**{**scan_kw(gb), "Dskip": gp["Dskip"]}, chunk_tokens=-1)
    assert np.array_equal(bits(y_full[:, 512:]), bits(y_blk))

    # block commit from the cached state == prefix state of prefix + block
    state = h_pre.clone()
    r2l.block_commit_state(state, gb["x"], gb["dt"], gb["Bm"], gb["A"], chunk_tokens=chunk)
    h_full_ref = oracle.prefix_scan_state(full.x, full.dt, full.Bm, full.A,
                                          seq_offsets=full.offsets)
    check_state(state, h_full_ref, "committed state")
    h_full = r2l.prefix_scan_state(gf["x"], gf["dt"], gf["Bm"], gf["A"], chunk_tokens=chunk)
    if chunk == -1:  # one plan, same per-token arithmetic: equal bit for bit
        assert np.array_equal(bits(state), bits(h_full))
    else:
        assert rel_err(host(state), host(h_full)) <= STATE_TOL

    # forward continuation of the block resumed from the cached state == the
    # full forward scan on the block's rows
    h_c, y_c = r2l.prefix_scan_state(gb["x"], gb["dt"], gb["Bm"], gb["A"], h_in=h_pre,
                                     Cm=gb["Cm"], Dskip=gp["Dskip"], chunk_tokens=-1)
    h_f, y_f = r2l.prefix_scan_state(gf["x"], gf["dt"], gf["Bm"], gf["A"], Cm=gf["Cm"],
                                     Dskip=gp["Dskip"], chunk_tokens=-1)
    if chunk == -1:  # the cached state came from the same unchunked plan
        assert np.array_equal(bits(y_c), bits(y_f[:, 512:]))
        assert np.array_equal(bits(h_c), bits(h_f))
    else:
        assert rel_err(host(y_c), host(y_f[:, 512:])) <= TOL["f32"]
    ref_f = oracle_scan(full, reverse=False, want_h_out=True)
    check_y(flat(y_f), ref_f["y"], "f32", "forward readout")
    check_state(h_c, ref_f["h_out"], "resumed state")
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# bit-exact classes
# ---------------------------------------------------------------------------
def unit_sum_inputs(lengths, D, dtype, seed):
    """A = 0, Delta = 1, Dskip = 0, only state 0 fed and read: y is a suffix sum."""
    r = np.random.default_rng(seed)
    tok = int(np.sum(lengths))
    lo = 2 if dtype == "bf16" else 8
    x = r.integers(-lo, lo + 1, (tok, D)).astype(np.float32)
    Bm = np.zeros((tok, 16), np.float32)
    Cm = np.zeros((tok, 16), np.float32)
    Bm[:, 0] = 1.0
    Cm[:, 0] = 1.0
    return synth.ScanInputs(dtype, np.asarray(lengths, np.int64), synth.offsets(lengths), x,
                            np.ones((tok, D), np.float32), Bm, Cm, np.zeros((D, 16), np.float32),
                            np.zeros(D, np.float32))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("split", [1, 2, 4])
@pytest.mark.parametrize("lengths", [[40] * 3, [5, 0, 1, 64, 17, 3, 0]])
def test_index_and_flip_bit_exact(gpu, dtype, split, lengths):
    D = 70  # a partial channel tile
    inp = unit_sum_inputs(lengths, D, dtype, len(lengths) + split)
    dense = len(set(lengths)) == 1
    g = on_gpu(inp, dense=dense)
    kw = scan_kw(g)
    rev = flat(r2l.r2l_scan(**kw, delta_softplus=False, state_split=split, chunk_tokens=-1))
    fwd_h, fwd = r2l.prefix_scan_state(kw["x"], kw["dt"], kw["Bm"], kw["A"], Cm=kw["Cm"],
                                       Dskip=kw["Dskip"], delta_softplus=False, state_split=split,
                                       chunk_tokens=-1, cu_seqlens=kw.get("cu_seqlens"),
                                       max_seqlen=kw.get("max_seqlen"))
    fwd = flat(fwd)
    rev_h, fwd_hh = host(rev), host(fwd)
    for b in range(inp.batch):
        seg = inp.rows(b)
        xs = inp.x[seg].astype(np.float64)
        assert np.array_equal(rev_h[seg], np.cumsum(xs[::-1], 0)[::-1]), b
        assert np.array_equal(fwd_hh[seg], np.cumsum(xs, 0)), b
        assert np.array_equal(host(fwd_h)[b, :, 0], xs.sum(0)), b
        assert not np.any(host(fwd_h)[b, :, 1:])
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gate_zero_returns_residual_bits(gpu, dtype):
    inp = synth.scan_inputs(11, [48] * 4, D=192, dtype=dtype)
    g = on_gpu(inp)
    res = torch.randn_like(g["x"])
    res.view(-1)[0] = -0.0
    res.view(-1)[5] = float("nan")
    res.view(-1)[7] = float("-inf")
    x = g["x"].clone()
    x.view(-1)[3 * 192 + 17] = float("inf")  # y turns non-finite in that channel
    out = r2l.r2l_scan(**{**scan_kw(g), "x": x}, res=res, s=0.0)
    assert np.array_equal(bits(out), bits(res))
    y = r2l.r2l_scan(**{**scan_kw(g), "x": x})
    assert not torch.isfinite(y.float()).all()
    # and in place: out is the residual itself
    res2 = res.clone()
    r2l.r2l_scan(**{**scan_kw(g), "x": x}, res=res2, s=0.0, out=res2)
    assert np.array_equal(bits(res2), bits(res))
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gate_zero_state_and_strided_copy(gpu, dtype):
    """s == 0 runs no readout: h_out comes from the state-only scan and equals,
    bit for bit, the state of the same call with the gate open; the residual
    is copied row by row into a strided out, leaving the padding alone."""
    inp = synth.scan_inputs(21, [40] * 3, D=72, dtype=dtype)
    g = on_gpu(inp)
    h0 = dev32(synth.initial_state(21, 3, 72, 16))
    h_open, h_closed = torch.empty_like(h0), torch.empty_like(h0)
    r2l.r2l_scan(**scan_kw(g), res=g["x"], s=0.5, h_in=h0, h_out=h_open, chunk_tokens=-1)
    out = r2l.r2l_scan(**scan_kw(g), res=g["x"], s=0.0, h_in=h0, h_out=h_closed, chunk_tokens=-1)
    assert np.array_equal(bits(h_closed), bits(h_open))
    assert np.array_equal(bits(out), bits(g["x"]))
    check_state(h_closed, oracle_scan(inp, h_in=synth.initial_state(21, 3, 72, 16),
                                      want_h_out=True)["h_out"])
    # strided residual and strided out (padded rows), dense batches
    wide_r = torch.full((3, 40, 100), 3.0, dtype=g["x"].dtype, device="cuda")
    wide_r[:, :, 10:82] = g["x"]
    wide_o = torch.full((3, 40, 90), 7.0, dtype=g["x"].dtype, device="cuda")
    r2l.r2l_scan(**scan_kw(g), res=wide_r[:, :, 10:82], s=0.0, out=wide_o[:, :, 5:77])
    assert np.array_equal(bits(wide_o[:, :, 5:77].contiguous()), bits(g["x"]))
    assert (wide_o[:, :, :5] == 7.0).all() and (wide_o[:, :, 77:] == 7.0).all()
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("split", [1, 4])
def test_reverse_equals_forward_on_flipped_input(gpu, dtype, split):
    inp = synth.scan_inputs(12, [75] * 3, D=130, dtype=dtype)
    g = on_gpu(inp)
    h0 = dev32(synth.initial_state(12, 3, 130, 16))
    hr = torch.empty_like(h0)
    yr = r2l.r2l_scan(**scan_kw(g), h_in=h0, h_out=hr, state_split=split, chunk_tokens=-1)
    fl = {k: (v.flip(1).contiguous() if k in ("x", "dt", "Bm", "Cm") else v)
          for k, v in g.items()}
    hf, yf = r2l.prefix_scan_state(fl["x"], fl["dt"], fl["Bm"], fl["A"], Cm=fl["Cm"],
                                   Dskip=fl["Dskip"], h_in=h0, state_split=split, chunk_tokens=-1)
    assert np.array_equal(bits(yr), bits(yf.flip(1).contiguous()))
    assert np.array_equal(bits(hr), bits(hf))
    torch.cuda.synchronize()


def test_chunked_reverse_resume_bit_exact(gpu):
    inp = synth.scan_inputs(13, [96] * 2, D=256)
    g = on_gpu(inp)
    hfull = torch.empty((2, 256, 16), device="cuda")
    yfull = r2l.r2l_scan(**scan_kw(g), h_out=hfull, chunk_tokens=-1)
    right = {k: (v[:, 40:] if k in ("x", "dt", "Bm", "Cm") else v) for k, v in g.items()}
    left = {k: (v[:, :40] if k in ("x", "dt", "Bm", "Cm") else v) for k, v in g.items()}
    hmid = torch.empty_like(hfull)
    yr = r2l.r2l_scan(**scan_kw(right), h_out=hmid, chunk_tokens=-1)
    hl = torch.empty_like(hfull)
    yl = r2l.r2l_scan(**scan_kw(left), h_in=hmid, h_out=hl, chunk_tokens=-1)
    assert np.array_equal(bits(torch.cat([yl, yr], 1)), bits(yfull))
    assert np.array_equal(bits(hl), bits(hfull))
    torch.cuda.synchronize()


def test_repeat_launches_are_identical(gpu):
    inp = synth.scan_inputs(14, [200] * 4, D=512, dtype="bf16")
    g = on_gpu(inp)
    a = r2l.r2l_scan(**scan_kw(g), chunk_tokens=64)
    for _ in range(3):
        b = r2l.r2l_scan(**scan_kw(g), chunk_tokens=64)
        assert np.array_equal(bits(a), bits(b))
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# chunked plans (the carry), with inputs whose memory outlives a chunk
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("chunk", [32, 100, 257])
def test_chunked_plans_carry_state(gpu, dtype, chunk):
    lengths = [700, 1, 0, 333, 64, 1025]
    inp = synth.scan_inputs(15, lengths, D=96, dtype=dtype, dt_mean=-6.0)
    g = on_gpu(inp, dense=False)
    h0 = synth.initial_state(15, len(lengths), 96, 16)
    ref = oracle_scan(inp, h_in=h0, want_h_out=True)
    # without the carry the answer would be far off: the test exercises it
    nocarry = []
    for b, L in enumerate(lengths):
        seg = inp.subset([b])
        parts = []
        for c0 in range(0, L, chunk):
            c1 = min(L, c0 + chunk)
            rows = slice(L - c1, L - c0)  # reverse scan: chunk c covers the c-th block from the right
            sub = synth.ScanInputs(inp.dtype, np.array([c1 - c0]), synth.offsets([c1 - c0]),
                                   seg.x[rows], seg.dt[rows], seg.Bm[rows], seg.Cm[rows], seg.A,
                                   seg.Dskip)
            parts.append((rows, oracle_scan(sub)["y"]))
        yb = np.zeros((L, 96))
        for rows, y in parts:
            yb[rows] = y
        nocarry.append(yb)
    assert rel_err(np.concatenate(nocarry), ref["y"]) > 10 * TOL[dtype]

    h_in = dev32(h0)
    h_out = torch.empty_like(h_in)
    y = r2l.r2l_scan(**scan_kw(g), h_in=h_in, h_out=h_out, chunk_tokens=chunk)
    check_y(y, ref["y"], dtype)
    check_state(h_out, ref["h_out"])

    fref = oracle_scan(inp, reverse=False, h_in=h0, want_h_out=True)
    hp = r2l.prefix_scan_state(g["x"], g["dt"], g["Bm"], g["A"], cu_seqlens=g["cu_seqlens"],
                               max_seqlen=g["max_seqlen"], h_in=h_in, chunk_tokens=chunk)
    check_state(hp, fref["h_out"], "chunked prefix state")
    st = h_in.clone()
    r2l.block_commit_state(st, g["x"], g["dt"], g["Bm"], g["A"], cu_seqlens=g["cu_seqlens"],
                           max_seqlen=g["max_seqlen"], chunk_tokens=chunk)
    check_state(st, fref["h_out"], "chunked commit")
    hy, yf = r2l.prefix_scan_state(g["x"], g["dt"], g["Bm"], g["A"], cu_seqlens=g["cu_seqlens"],
                                   max_seqlen=g["max_seqlen"], h_in=h_in, Cm=g["Cm"],
                                   Dskip=g["Dskip"], chunk_tokens=chunk)
    check_y(yf, fref["y"], dtype, "chunked forward readout")
    check_state(hy, fref["h_out"])
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("res", ["none", "x", "separate", "x_s0", "in_place", "in_place_s0"])
def test_chunked_readout_plans(gpu, dtype, res):
    """Chunked readout plans write chunk 0 in the chunk pass (from the call's
    initial state) and the other chunks in the readout pass; without h_out the
    chunk pass skips each sequence's last chunk. Every combination of h_in,
    h_out and residual form, on sequences shorter than, equal to and longer
    than a chunk, and empty ones."""
    lengths = [300, 1, 0, 64, 65, 129, 40, 192]
    D, chunk = 80, 64
    inp = synth.scan_inputs(19, lengths, D=D, dtype=dtype, dt_mean=-4.0)
    g = on_gpu(inp, dense=False)
    h0 = synth.initial_state(19, len(lengths), D, 16)
    s = 0.0 if res.endswith("_s0") else 0.3
    res_np = {"none": None, "separate": synth.scan_inputs(20, lengths, D=D, dtype=dtype).x}.get(
        res, inp.x)
    for with_hin in (False, True):
        for with_hout in (False, True):
            ref = oracle_scan(inp, res=res_np, s=s, h_in=h0 if with_hin else None,
                              want_h_out=with_hout, want_out=res_np is not None)
            x = g["x"].clone()
            kw = dict(scan_kw(g), x=x, chunk_tokens=chunk)
            if with_hin:
                kw["h_in"] = dev32(h0)
            if with_hout:
                kw["h_out"] = torch.full((len(lengths), D, 16), float("nan"), device="cuda")
            if res_np is not None:
                kw.update(res=x if res != "separate" else dev(res_np, dtype), s=s)
            if res.startswith("in_place"):
                kw["out"] = x
            out = r2l.r2l_scan(**kw)
            what = "%s h_in=%d h_out=%d" % (res, with_hin, with_hout)
            if res_np is None:
                check_y(out, ref["y"], dtype, what)
            elif s == 0.0:
                assert np.array_equal(bits(out), bits(dev(res_np, dtype))), what
            else:
                check_y(out, ref["out"], dtype, what)
            if with_hout:
                check_state(kw["h_out"], ref["h_out"], what)
            plan = r2l.bind("r2l_scan", **{**kw, "out": out}).plan()
            if s != 0.0:
                assert plan["chunked"] and plan["launches"] == 3
            else:   # no readout: the state-only plan when h_out is wanted, then the copy
                assert plan["launches"] == (2 if with_hout else 0) + (res == "x_s0")
    torch.cuda.synchronize()


def test_graph_replays_match_eager(gpu):
    """Calls captured once in a hipGraph (the benchmark replays its steps this
    way) give the eager results on every replay, with eager work between the
    replays: a chunked plan (chunk pass, carry, readout pass through the bound
    workspace), a gated in-place hook and an s == 0 residual copy."""
    lengths = [300, 17, 0, 129]
    inp = synth.scan_inputs(22, lengths, D=96, dtype="bf16", dt_mean=-4.0)
    g = on_gpu(inp, dense=False)
    h0 = dev32(synth.initial_state(22, len(lengths), 96, 16))
    x_hook = g["x"].clone()
    res = torch.randn_like(g["x"])
    bufs = {"y": torch.empty_like(g["x"]), "h": torch.empty_like(h0),
            "copy": torch.empty_like(g["x"])}
    calls = [r2l.bind("r2l_scan", **scan_kw(g), h_in=h0, h_out=bufs["h"], out=bufs["y"],
                      chunk_tokens=64),
             r2l.bind("r2l_scan", **{**scan_kw(g), "x": x_hook}, res=x_hook, s=0.3, out=x_hook),
             r2l.bind("r2l_scan", **scan_kw(g), res=res, s=0.0, out=bufs["copy"])]
    assert calls[0].plan()["launches"] == 3 and calls[2].plan()["launches"] == 1
    x_start = x_hook.clone()
    for c in calls:
        c.launch()
    eager = {k: bits(v) for k, v in bufs.items()}
    eager["hook"] = bits(x_hook)

    x_hook.copy_(x_start)
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            for c in calls:
                c.launch(stream.cuda_stream)
    torch.cuda.synchronize()
    for rep in range(4):
        for v in bufs.values():          # eager work between replays
            v.fill_(float("nan"))
        x_hook.copy_(x_start)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in bufs.items():
            assert np.array_equal(bits(v), eager[k]), "replay %d: %s" % (rep, k)
        assert np.array_equal(bits(x_hook), eager["hook"]), "replay %d: hook" % rep
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------
def test_empty_batch_and_empty_sequences(gpu):
    A = torch.full((32, 16), -1.0, device="cuda")
    x = torch.zeros((0, 32), device="cuda")
    e16 = torch.zeros((0, 16), device="cuda")
    cu = torch.zeros(1, dtype=torch.int32, device="cuda")
    r2l.r2l_scan(x, x, e16, e16, A, cu_seqlens=cu, max_seqlen=0)
    # three empty sequences: h_out = h_in (or zero)
    cu = torch.zeros(4, dtype=torch.int32, device="cuda")
    h0 = torch.randn((3, 32, 16), device="cuda")
    h1 = torch.full_like(h0, 7.0)
    r2l.r2l_scan(x, x, e16, e16, A, cu_seqlens=cu, max_seqlen=0, h_in=h0, h_out=h1)
    assert torch.equal(h1, h0)
    r2l.r2l_scan(x, x, e16, e16, A, cu_seqlens=cu, max_seqlen=0, h_out=h1)
    assert not h1.any()
    # dense seqlen 0
    x3 = torch.zeros((3, 0, 32), device="cuda")
    b3 = torch.zeros((3, 0, 16), device="cuda")
    hp = r2l.prefix_scan_state(x3, x3, b3, A, h_in=h0)
    assert torch.equal(hp, h0)
    torch.cuda.synchronize()


def test_maximum_dim(gpu):
    """dim at the largest value the library takes (65535 * 16 channels: the
    carry grid's y limit), with a chunked state-only call that uses that grid."""
    D = 65535 * 16
    inp = synth.scan_inputs(23, [3, 5], D=D)
    g = on_gpu(inp, dense=False)
    h0 = synth.initial_state(23, 2, D, 16)
    ref = oracle_scan(inp, h_in=h0, want_h_out=True)
    h = torch.empty((2, D, 16), device="cuda")
    y = r2l.r2l_scan(**scan_kw(g), h_in=dev32(h0), h_out=h)
    check_y(y, ref["y"], "f32", "max dim y")
    check_state(h, ref["h_out"], "max dim state")
    fref = oracle_scan(inp, reverse=False, h_in=h0, want_h_out=True)
    hp = r2l.prefix_scan_state(g["x"], g["dt"], g["Bm"], g["A"], cu_seqlens=g["cu_seqlens"],
                               max_seqlen=g["max_seqlen"], h_in=dev32(h0), chunk_tokens=2)
    check_state(hp, fref["h_out"], "max dim chunked prefix state")
    torch.cuda.synchronize()


def test_million_token_sequence(gpu):
    """One sequence of 2^20 tokens: the planner cuts it into thousands of
    chunks (a long carry per lane)."""
    L, D = 1 << 20, 16
    inp = synth.scan_inputs(24, [L], D=D, dtype="bf16", dt_mean=-5.0)
    g = on_gpu(inp, dense=False)
    ref = oracle_scan(inp, want_h_out=True)
    h = torch.empty((1, D, 16), device="cuda")
    kw = dict(scan_kw(g), h_out=h)
    plan = r2l.bind("r2l_scan", **kw, out=torch.empty_like(g["x"])).plan()
    assert plan["chunked"] and plan["chunks"] > 1000
    y = r2l.r2l_scan(**kw)
    check_y(y, ref["y"], "bf16", "2^20 tokens y")
    check_state(h, ref["h_out"], "2^20 tokens state")
    fref = oracle_scan(inp, reverse=False, want_h_out=True)
    hp = r2l.prefix_scan_state(g["x"], g["dt"], g["Bm"], g["A"], cu_seqlens=g["cu_seqlens"],
                               max_seqlen=g["max_seqlen"])
    check_state(hp, fref["h_out"], "2^20 tokens prefix state")
    torch.cuda.synchronize()


def test_many_short_sequences(gpu):
    """60 000 ragged sequences of 0 to 3 tokens (one block each)."""
    rng = np.random.default_rng(25)
    lengths = rng.integers(0, 4, size=60_000)
    inp = synth.scan_inputs(25, lengths, D=16)
    g = on_gpu(inp, dense=False)
    ref = oracle_scan(inp, want_h_out=True)
    h = torch.empty((len(lengths), 16, 16), device="cuda")
    y = r2l.r2l_scan(**scan_kw(g), h_out=h)
    check_y(y, ref["y"], "f32", "short sequences y")
    check_state(h, ref["h_out"], "short sequences state")
    torch.cuda.synchronize()


@pytest.mark.parametrize("D", [1, 37, 100, 320])
@pytest.mark.parametrize("split", [1, 2, 4])
def test_channel_tile_tails(gpu, D, split):
    inp = synth.scan_inputs(16, [19, 70], D=D)
    g = on_gpu(inp, dense=False)
    ref = oracle_scan(inp, want_h_out=True)
    h = torch.empty((2, D, 16), device="cuda")
    y = r2l.r2l_scan(**scan_kw(g), h_out=h, state_split=split)
    check_y(y, ref["y"], "f32")
    check_state(h, ref["h_out"])
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_strided_and_in_place(gpu, dtype):
    inp = synth.scan_inputs(17, [33] * 5, D=200, dtype=dtype)
    ref = oracle_scan(inp, res=inp.x, s=0.3, want_out=True)
    g = on_gpu(inp)
    # token rows with padding between them
    wide = torch.zeros((5, 33, 264), dtype=g["x"].dtype, device="cuda")
    wide[:, :, 8:208] = g["x"]
    xs = wide[:, :, 8:208]
    dts = torch.zeros_like(wide)
    dts[:, :, 8:208] = g["dt"]
    out = r2l.r2l_scan(xs, dts[:, :, 8:208], g["Bm"], g["Cm"], g["A"], g["Dskip"], res=xs, s=0.3)
    check_y(flat(out), ref["out"], dtype, "strided out")
    # in place on the hidden states (out is x and res): same bits as out of place
    r2l.r2l_scan(xs, dts[:, :, 8:208], g["Bm"], g["Cm"], g["A"], g["Dskip"], res=xs, s=0.3,
                 out=xs)
    assert np.array_equal(bits(xs.contiguous()), bits(out))
    assert not wide[:, :, :8].any() and not wide[:, :, 208:].any()
    torch.cuda.synchronize()


def test_plans_agree(gpu):
    inp = synth.scan_inputs(18, [300] * 2, D=256, dtype="f32")
    g = on_gpu(inp)
    ref = oracle_scan(inp, want_h_out=True)
    for split in (1, 2, 4):
        for chunk in (-1, 64, 128):
            h = torch.empty((2, 256, 16), device="cuda")
            y = r2l.r2l_scan(**scan_kw(g), h_out=h, state_split=split, chunk_tokens=chunk)
            check_y(flat(y), ref["y"], "f32", "split %d chunk %d" % (split, chunk))
            check_state(h, ref["h_out"])
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# full-size workloads
# ---------------------------------------------------------------------------
def test_denoise_hooks_bf16(gpu):
    s = synth.denoise_gates()
    for hook in (0, 6):
        inp = synth.denoise_hook_inputs(hook)
        ref = oracle_scan(inp, res=inp.x, s=float(s[hook]), want_out=True)
        g = on_gpu(inp)
        y = r2l.r2l_scan(**scan_kw(g))
        check_y(flat(y), ref["y"], "bf16", "hook %d y" % hook)
        x = g["x"].clone()
        r2l.r2l_scan(**{**scan_kw(g), "x": x}, res=x, s=float(s[hook]), out=x)
        check_y(flat(x), ref["out"], "bf16", "hook %d out" % hook)
    torch.cuda.synchronize()


def test_l2r_ablation_hooks_bf16(gpu):
    """The L2R-Mamba ablation at the denoising hook shape: forward scan with
    readout and gated residual in place, through prefix_scan_state."""
    s = synth.denoise_gates()
    for hook in (0, 6):
        inp = synth.denoise_hook_inputs(hook)
        ref = oracle_scan(inp, reverse=False, res=inp.x, s=float(s[hook]), want_out=True,
                          want_h_out=True)
        g = on_gpu(inp)
        x = g["x"].clone()
        h = torch.empty((64, 2048, 16), device="cuda")
        r2l.prefix_scan_state(x, g["dt"], g["Bm"], g["A"], Cm=g["Cm"], Dskip=g["Dskip"], res=x,
                              s=float(s[hook]), out=x, h_out=h)
        check_y(flat(x), ref["out"], "bf16", "hook %d forward out" % hook)
        check_state(h, ref["h_out"], "hook %d forward state" % hook)
    torch.cuda.synchronize()


def test_prefill_bf16_sampled(gpu):
    inp = synth.prefill_inputs()
    g = on_gpu(inp)
    y = r2l.r2l_scan(**scan_kw(g))
    torch.cuda.synchronize()
    for b in (0, 7):
        sub = inp.subset([b])
        ref = oracle_scan(sub)
        check_y(y[b], ref["y"], "bf16", "sequence %d" % b)


def test_ragged_serving_bf16_sampled(gpu):
    blk = synth.ragged_block_inputs()
    com = synth.ragged_commit_inputs()
    gb, gc = on_gpu(blk, dense=False), on_gpu(com, dense=False)
    y = r2l.r2l_scan(**scan_kw(gb))
    h0 = synth.initial_state(synth.RAGGED.key, 256, 4096, 16)
    state = dev32(h0)
    r2l.block_commit_state(state, gc["x"], gc["dt"], gc["Bm"], gc["A"],
                           cu_seqlens=gc["cu_seqlens"], max_seqlen=gc["max_seqlen"])
    torch.cuda.synchronize()
    yh, sh = host(y), host(state)
    for b in (0, 1, 77, 128, 255):
        ref = oracle_scan(blk.subset([b]))
        seg = blk.rows(b)
        check_y(y[seg], ref["y"], "bf16", "block %d" % b)
        c = com.subset([b])
        href = oracle.block_commit_state(h0[b:b + 1], c.x, c.dt, c.Bm, c.A, seq_offsets=c.offsets)
        check_state(state[b:b + 1], href, "commit %d" % b)
    del yh, sh


def test_ragged_prefix_prefill_subset(gpu):
    seqs = [0, 5, 17, 99, 200, 255]
    pre = synth.ragged_prefix_inputs(seqs=seqs)
    g = on_gpu(pre, dense=False)
    h = r2l.prefix_scan_state(g["x"], g["dt"], g["Bm"], g["A"], cu_seqlens=g["cu_seqlens"],
                              max_seqlen=g["max_seqlen"])
    ref = oracle.prefix_scan_state(pre.x, pre.dt, pre.Bm, pre.A, seq_offsets=pre.offsets)
    check_state(h, ref, "prefill prefix states")
    torch.cuda.synchronize()


def _device_draws(seed, tok, D, dt_mean):
    """Seeded inputs drawn on the GPU (the distributions of synth, dt ~ N(dt_mean,
    0.5)) for the full-size plans, whose inputs are too large to draw on the host;
    the oracle reads back the sampled sequences."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    bf = torch.bfloat16
    return {"x": torch.randn((tok, D), generator=g, device="cuda").to(bf),
            "dt": (torch.randn((tok, D), generator=g, device="cuda") * 0.5 + dt_mean).to(bf),
            "Bm": torch.randn((tok, 16), generator=g, device="cuda").to(bf),
            "Cm": torch.randn((tok, 16), generator=g, device="cuda").to(bf),
            "A": -(torch.arange(16, device="cuda", dtype=torch.float32) + 1).repeat(D, 1),
            "Dskip": torch.randn((D,), generator=g, device="cuda")}


def _ulp_factor(got, ref):
    """Worst element in units of (one bf16 ulp of ref + 1e-5 * max|ref|)."""
    ref = np.asarray(ref, dtype=np.float64)
    slack = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 2.0 ** -126))) - 7) + \
        1e-5 * np.max(np.abs(ref))
    return float(np.max(np.abs(np.asarray(got, dtype=np.float64) - ref) / slack))


def test_prefill_long_memory_full_plan(gpu):
    """The prefill shape (8 x 4096 x 4096, bf16) with long-memory inputs (dt ~
    N(-6, 0.5): Delta ~ 0.0025, state memory of hundreds of tokens) under the
    planner's own plan (9 chunks of 456 tokens: chunk pass, carry, readout pass);
    sampled sequences against the oracle. A reverse scan that dropped the carry
    into the chunks left of the rightmost would be off by more than ten times the
    element bound there."""
    B, L, D = 8, 4096, 4096
    g = _device_draws(3101, B * L, D, -6.0)
    view = {k: (g[k].view(B, L, -1) if k in ("x", "dt", "Bm", "Cm") else g[k]) for k in g}
    y = torch.empty_like(view["x"])
    call = r2l.bind("r2l_scan", out=y, **view)
    plan = call.plan()
    assert plan["chunked"] and plan["chunks"] == 9 and plan["chunk_tokens"] == 456, plan
    call.launch()
    torch.cuda.synchronize()
    A, Ds = g["A"].cpu().numpy(), g["Dskip"].cpu().numpy()
    for b in (0, 7):
        rows = slice(b * L, (b + 1) * L)
        x, dt, Bm, Cm = (g[k][rows].float().cpu().numpy() for k in ("x", "dt", "Bm", "Cm"))
        ref = oracle.selective_scan(x, dt, Bm, Cm, A, Ds, reverse=True,
                                    seq_offsets=np.array([0, L]))
        check_y(y[b], ref["y"], "bf16", "long-memory sequence %d" % b)
        n = L - 456    # left of the rightmost chunk, scanned from zero: no carry
        nc = oracle.selective_scan(x[:n], dt[:n], Bm[:n], Cm[:n], A, Ds, reverse=True,
                                   seq_offsets=np.array([0, n]))
        assert _ulp_factor(nc["y"], ref["y"][:n]) > 10.0


def test_ragged_prefix_prefill_full_plan(gpu):
    """The ragged prefix-state prefill at its full size (256 prefixes of
    U{256..8192} tokens, D = 4096, bf16: the benchmark's call and plan, chunks
    of at most 1024 tokens joined by the carry); the final states of sampled
    prefixes (the shortest, the longest, and spread ones) against the oracle."""
    lens = synth.ragged_prefix_lengths()
    off = synth.offsets(lens)
    D = 4096
    g = _device_draws(3102, int(off[-1]), D, -2.0)
    cu = torch.from_numpy(off.astype(np.int32)).cuda()
    h = torch.empty((len(lens), D, 16), dtype=torch.float32, device="cuda")
    call = r2l.bind("prefix_scan_state", x=g["x"], dt=g["dt"], Bm=g["Bm"], A=g["A"], h_out=h,
                    cu_seqlens=cu, max_seqlen=int(lens.max()))
    plan = call.plan()
    assert plan["chunked"] and plan["chunk_tokens"] <= 1024, plan
    call.launch()
    torch.cuda.synchronize()
    A = g["A"].cpu().numpy()
    for b in sorted({0, 100, 255, int(np.argmin(lens)), int(np.argmax(lens))}):
        rows = slice(int(off[b]), int(off[b + 1]))
        x, dt, Bm = (g[k][rows].float().cpu().numpy() for k in ("x", "dt", "Bm"))
        ref = oracle.prefix_scan_state(x, dt, Bm, A, seq_offsets=np.array([0, x.shape[0]]))
        check_state(h[b:b + 1], ref, "prefix %d (%d tokens)" % (b, lens[b]))
