"""r2l_scan_noalloc (through the C ABI) against r2l_scan with a caller
workspace: the same plan and kernels, so the outputs and final states must be
the same bits; the first case is also held to the fp64 oracle at the parity
bar. The calls without allocation run back to back, the second on a smaller
input, so the second finds the first one's data in the shared scratch array.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import reverse_mamba_selective_amd as r2l
import synth
from gpu_util import bits, check_state, check_y, dev, dev32, gpu  # noqa: F401

pytestmark = pytest.mark.gpu


def _inputs(seed, lengths, D, dtype, dense):
    inp = synth.scan_inputs(seed, lengths, D=D, dtype=dtype, dt_mean=-4.0)
    B = inp.batch
    shaped = (lambda t: t.view(B, int(lengths[0]), -1)) if dense else (lambda t: t)
    x = shaped(dev(inp.x, dtype))
    kw = dict(dt=shaped(dev(inp.dt, dtype)), Bm=shaped(dev(inp.Bm, dtype)),
              Cm=shaped(dev(inp.Cm, dtype)), A=dev32(inp.A), Dskip=dev32(inp.Dskip))
    if not dense:
        kw.update(cu_seqlens=torch.from_numpy(inp.offsets.astype(np.int32)).cuda(),
                  max_seqlen=int(inp.lengths.max()))
    return inp, x, kw


CASES = [
    # (seed, lengths, D, dtype, dense): the planner chunks the first two
    (71, [3000, 1, 2000, 0, 517], 128, "bf16", False),
    (72, [4096, 4096], 512, "bf16", True),
    (73, [700, 33, 5], 64, "f32", False),
    (74, [32] * 8, 256, "bf16", True),     # no chunking: no scratch at all
]


def test_noalloc_matches_r2l_scan(gpu):
    sets = []
    for seed, lengths, D, dtype, dense in CASES:
        inp, x, kw = _inputs(seed, lengths, D, dtype, dense)
        B = inp.batch
        h_in = dev32(synth.initial_state(seed, B, D, 16))
        need = r2l.workspace_size("r2l_scan", x, kw["A"], cu_seqlens=kw.get("cu_seqlens"),
                                  max_seqlen=kw.get("max_seqlen"))
        assert need <= r2l.NOALLOC_SCRATCH_BYTES
        h_ref = torch.empty((B, D, 16), dtype=torch.float32, device="cuda")
        ref = r2l.r2l_scan(x, **kw, h_in=h_in, h_out=h_ref, res=x, s=0.3)
        sets.append((inp, x, kw, h_in, h_ref, ref, need))
    assert sets[0][6] > 0 and sets[1][6] > 0 and sets[3][6] == 0
    torch.cuda.synchronize()
    got = []
    for inp, x, kw, h_in, _, ref, _ in sets:   # back to back, the scratch shared
        out = torch.empty_like(ref)
        h = torch.empty((inp.batch, x.shape[-1], 16), dtype=torch.float32, device="cuda")
        r2l.r2l_scan_noalloc(x, **kw, out=out, h_in=h_in, h_out=h, res=x, s=0.3)
        got.append((out, h))
    torch.cuda.synchronize()
    for (inp, x, kw, h_in, h_ref, ref, _), (out, h) in zip(sets, got):
        assert np.array_equal(bits(out), bits(ref)), "out differs from r2l_scan's"
        assert np.array_equal(bits(h), bits(h_ref)), "h_out differs from r2l_scan's"
    inp, x, kw, h_in, _, _, _ = sets[0]
    h0 = synth.initial_state(CASES[0][0], inp.batch, CASES[0][2], 16)
    want = oracle.selective_scan(inp.x, inp.dt, inp.Bm, inp.Cm, inp.A, inp.Dskip, reverse=True,
                                 seq_offsets=inp.offsets, h_in=h0, want_h_out=True, res=inp.x,
                                 s=0.3, want_out=True)
    check_y(got[0][0].reshape(-1, CASES[0][2]), want["out"], "bf16", "out")
    check_state(got[0][1], want["h_out"], "h_out")


def test_noalloc_twice_in_a_row_smaller_second(gpu):
    """Two calls without allocation in a row on one stream, the second on a
    smaller chunked input, each equal to r2l_scan's bits."""
    big = _inputs(75, [2500, 1800], 256, "bf16", False)
    small = _inputs(76, [900, 300, 1], 128, "bf16", False)
    refs, outs = [], []
    for inp, x, kw in (big, small):
        refs.append(r2l.r2l_scan(x, **kw, res=None))
    torch.cuda.synchronize()
    for inp, x, kw in (big, small):
        out = torch.empty_like(x)
        outs.append(r2l.r2l_scan_noalloc(x, **kw, out=out))
    torch.cuda.synchronize()
    for r, o in zip(refs, outs):
        assert np.array_equal(bits(o), bits(r))


def test_noalloc_refuses_plans_beyond_the_scratch(gpu):
    inp, x, kw = _inputs(77, [40000], 1024, "bf16", False)
    kw["chunk_tokens"] = 64     # 625 chunks of 1024 channels: > 64 MiB of carry data
    need = r2l.workspace_size("r2l_scan", x, kw["A"], cu_seqlens=kw["cu_seqlens"],
                              max_seqlen=kw["max_seqlen"], chunk_tokens=64)
    assert need > r2l.NOALLOC_SCRATCH_BYTES
    out = torch.full_like(x, 7.0)
    with pytest.raises(r2l.R2LError) as e:
        r2l.r2l_scan_noalloc(x, **kw, out=out)
    assert e.value.status == r2l._abi.R2L_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()), "a refused call wrote its output"
