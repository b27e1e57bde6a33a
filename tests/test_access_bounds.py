"""Every memory access the kernels would make, replayed on the CPU.

``r2l_check_access`` runs a call's argument checks, plan and launch list and
walks the kernels' own index math (scan_geometry.h) over every block, lane,
token and staging slot, with fake device addresses that are only compared,
never dereferenced. Each case here must come back with every access inside
the buffer its base pointer belongs to. This runs before any kernel change
goes to a GPU.
"""
import random

import numpy as np
import pytest

from reverse_mamba_selective_amd import _abi

BASE = 0x7E0000000000
OPS = {"scan": _abi.R2L_OP_SCAN, "prefix": _abi.R2L_OP_PREFIX, "commit": _abi.R2L_OP_COMMIT}


class FakeHeap:
    """Page-aligned fake allocations separated by guard gaps; size 0 gives NULL,
    as torch does for an empty tensor."""

    def __init__(self):
        self.next = BASE

    def alloc(self, nbytes):
        if nbytes == 0:
            return None
        p = self.next
        self.next += (nbytes + 4095) // 4096 * 4096 + 65536
        return p


def make_args(op, *, dtype="bf16", D=64, batch=None, seqlen=None, lengths=None, res="none",
              h_in=False, h_out=False, out=True, chunk=-1, split=0, pad_row=0, pad_batch=0,
              bc_shift=0, s=0.05):
    """A call with every buffer sized exactly as the layout says. bc_shift
    starts Bm and Cm that many elements into their allocation (which grows by
    as much), breaking the alignment of the staging's vector loads."""
    es = 2 if dtype == "bf16" else 4
    N = 16
    heap = FakeHeap()
    a = _abi.ScanArgs()
    a.dim, a.dstate = D, N
    a.dtype = _abi.R2L_DTYPE_BF16 if dtype == "bf16" else _abi.R2L_DTYPE_F32
    a.delta_softplus = 1
    a.chunk_tokens, a.state_split = chunk, split
    cu = None
    if lengths is not None:
        lengths = list(lengths)
        a.batch = len(lengths)
        cu = [0] + list(np.cumsum(lengths))
        a.total_tokens, a.max_seqlen = int(cu[-1]), max(lengths) if lengths else 0
        a.cu_seqlens = heap.alloc(4 * (a.batch + 1))
        tok = a.total_tokens

        def tensor(cols, lead=0):
            stride = cols + pad_row
            return offset(heap.alloc(((tok - 1) * stride + cols + lead) * es if tok else 0),
                          lead), stride, 0
    else:
        a.batch, a.seqlen = batch, seqlen
        tok = batch * seqlen

        def tensor(cols, lead=0):
            stride = cols + pad_row
            bstride = seqlen * stride + pad_batch
            ext = ((batch - 1) * bstride + (seqlen - 1) * stride + cols + lead) if tok else 0
            return offset(heap.alloc(ext * es), lead), stride, bstride if pad_batch else 0

    def offset(p, lead):   # `lead` elements into the allocation
        return p + lead * es if p is not None else None

    a.x, a.x_stride, a.x_batch_stride = tensor(D)
    a.dt, a.dt_stride, a.dt_batch_stride = tensor(D)
    a.Bm, a.Bm_stride, a.Bm_batch_stride = tensor(N, bc_shift)
    readout = op == "scan" or out
    if readout:
        a.Cm, a.Cm_stride, a.Cm_batch_stride = tensor(N, bc_shift)
        a.out, a.out_stride, a.out_batch_stride = tensor(D)
        a.Dskip = heap.alloc(4 * D)
        if res == "x":
            a.res, a.res_stride, a.res_batch_stride = a.x, a.x_stride, a.x_batch_stride
        elif res == "sep":
            a.res, a.res_stride, a.res_batch_stride = tensor(D)
        elif res == "sep_into_x":   # a separate residual, out is x
            a.res, a.res_stride, a.res_batch_stride = tensor(D)
            a.out, a.out_stride, a.out_batch_stride = a.x, a.x_stride, a.x_batch_stride
        elif res == "inplace":  # out is x is res
            a.res, a.res_stride, a.res_batch_stride = a.x, a.x_stride, a.x_batch_stride
            a.out, a.out_stride, a.out_batch_stride = a.x, a.x_stride, a.x_batch_stride
        a.s = s
    a.A = heap.alloc(4 * D * N)
    if h_in and op != "commit":
        a.h_in = heap.alloc(4 * a.batch * D * N)
    if h_out or op == "commit" or (op == "prefix" and (not out or tok == 0)):
        a.h_out = heap.alloc(4 * a.batch * D * N)
    need = _abi.workspace_size(OPS[op], a)
    if need:
        a.workspace, a.workspace_bytes = heap.alloc(need), need
    return a, cu


def check(op, **kw):
    a, cu = make_args(op, **kw)
    st, rep = _abi.check_access(OPS[op], a, cu)
    msg = rep.message.decode() or _abi.last_error()
    assert st == _abi.R2L_OK, "%s %s: %s" % (op, kw, msg)
    return rep


# ---- explicit edge cases -----------------------------------------------------
EDGE = [
    dict(lengths=[0, 0, 0], h_in=True, h_out=True),           # only empty sequences
    dict(lengths=[5, 0, 1, 64, 17, 3, 0], h_out=True),
    dict(lengths=[1]),
    dict(lengths=[65, 64, 63, 128, 129]),
    dict(batch=3, seqlen=0, h_in=True, h_out=True),           # dense, no token at all
    dict(batch=1, seqlen=1),
    dict(batch=2, seqlen=200, D=37),
    dict(batch=2, seqlen=97, D=1),
    dict(batch=4, seqlen=33, D=300, pad_row=8, pad_batch=40),  # padded rows and batches
    dict(lengths=[700, 1, 0, 333, 64, 1025], D=96, chunk=100, h_in=True, h_out=True),
    dict(lengths=[700, 1, 0, 333, 64, 1025], D=96, chunk=32, h_out=True),
    dict(batch=2, seqlen=300, D=256, chunk=64, h_out=True),
]


@pytest.mark.parametrize("op", ["scan", "prefix", "commit"])
@pytest.mark.parametrize("case", range(len(EDGE)))
@pytest.mark.parametrize("split", [1, 2, 4])
def test_edge_cases(op, case, split):
    kw = dict(EDGE[case])
    for res in (["none", "x", "sep", "inplace"] if op == "scan" else ["none"]):
        check(op, split=split, res=res, **kw)
    if op == "prefix":
        check(op, split=split, out=False, **kw)
        check(op, split=split, **{**kw, "out": True, "h_out": True})
    if op == "commit":
        check(op, split=split, out=False, **kw)


def test_random_plans():
    rng = random.Random(1234)
    for _ in range(300):
        op = rng.choice(["scan", "prefix", "commit"])
        kw = dict(dtype=rng.choice(["bf16", "f32"]), D=rng.choice([1, 5, 64, 100, 256, 513]),
                  split=rng.choice([0, 1, 2, 4]), chunk=rng.choice([-1, 0, 16, 33, 64, 200]),
                  h_in=rng.random() < 0.5, h_out=rng.random() < 0.5,
                  pad_row=rng.choice([0, 0, 1, 2, 8, 16]), bc_shift=rng.choice([0, 0, 0, 1, 2]))
        if rng.random() < 0.5:
            kw["lengths"] = [rng.choice([0, 1, 2, 31, 64, 65, 130, 300]) for _ in range(rng.randint(1, 6))]
        else:
            kw.update(batch=rng.randint(1, 5), seqlen=rng.choice([0, 1, 8, 63, 64, 65, 257]),
                      pad_batch=rng.choice([0, 0, 24]))
        if op == "scan":
            kw["res"] = rng.choice(["none", "x", "sep", "inplace"])
            kw["s"] = rng.choice([0.05, 0.05, 0.0])
        else:
            kw["out"] = rng.random() < 0.4
        check(op, **kw)


# ---- Bm/Cm staging: vector loads only where every row start is aligned -------
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("op", ["scan", "prefix"])
def test_staging_vector_choice(dtype, op):
    kw = dict(dtype=dtype, lengths=[70, 0, 130, 1], D=96, chunk=64, h_out=True)
    if op == "prefix":
        kw["out"] = False                  # state only: chunk pass and carry
    launches = 3 if op == "scan" else 2   # chunk pass, carry (, readout pass)
    assert check(op, **kw).vector_staging == launches - 1
    # row strides of 17 or 18 elements: rows on 2- or 4-byte boundaries only
    # (bf16), or on 4- or 8-byte ones (f32): element loads
    for pad in (1, 2):
        assert check(op, pad_row=pad, **kw).vector_staging == 0
    # base one element in: element loads
    assert check(op, bc_shift=1, **kw).vector_staging == 0
    # a row stride of 24 elements keeps 16-byte rows for bf16 and f32
    assert check(op, pad_row=8, **kw).vector_staging == launches - 1
    # dense batches: a batch stride off the alignment
    dense = dict(dtype=dtype, batch=3, seqlen=65, D=64, chunk=32, h_out=True, out=op == "scan")
    assert check(op, **dense).vector_staging == launches - 1
    assert check(op, pad_batch=1, **dense).vector_staging == 0


# ---- s == 0: the output is the residual; no readout runs -------------------
@pytest.mark.parametrize("layout", [
    dict(lengths=[5, 0, 1, 64, 17, 300]),
    dict(batch=3, seqlen=70, pad_row=8, pad_batch=40),
    dict(batch=2, seqlen=0)])
def test_gate_closed_plans(layout):
    kw = dict(D=96, s=0.0, **layout)
    tok = sum(layout.get("lengths", [])) or layout.get("batch", 0) * layout.get("seqlen", 0)
    copies = 1 if tok else 0
    # out == x == res: nothing to do at all
    assert check("scan", res="inplace", **kw).launches == 0
    # a new out: one row copy of the residual (x or a separate tensor)
    for res in ("x", "sep"):
        assert check("scan", res=res, **kw).launches == copies
        # the state is still scanned when h_out is wanted (state only), before the copy
        assert check("scan", res=res, h_out=True, h_in=True, **kw).launches == 1 + copies
        rep = check("scan", res=res, h_out=True, chunk=32, **kw)
        assert rep.launches == (2 if tok else 1) + copies
    assert check("scan", res="inplace", h_out=True, **kw).launches == 1
    a, _ = make_args("scan", res="x", **kw)
    assert _abi.workspace_size(_abi.R2L_OP_SCAN, a) == 0


# ---- the largest shapes the GPU tests run --------------------------------------
def test_maximum_size_shapes():
    D = 65535 * 16
    check("scan", lengths=[3, 5], D=D, dtype="f32", h_in=True, h_out=True, chunk=0)
    check("prefix", lengths=[3, 5], D=D, dtype="f32", h_in=True, out=False, chunk=2)
    rep = check("scan", lengths=[1 << 20], D=16, h_out=True, chunk=0)
    assert rep.launches == 3
    check("prefix", lengths=[1 << 20], D=16, out=False, chunk=0)
    lengths = np.random.default_rng(25).integers(0, 4, size=60_000)
    check("scan", lengths=lengths, D=16, h_out=True, chunk=0, dtype="f32")


# ---- the benchmarked shapes, at full size --------------------------------------
# (chunk=0: the plan the library picks, as the benchmark runs it)
def test_denoise_hook_shape():
    rep = check("scan", batch=64, seqlen=32, D=2048, res="x", chunk=0)
    assert rep.launches == 1 and rep.accesses > 0


def test_prefill_shape():
    rep = check("scan", batch=8, seqlen=4096, D=4096, chunk=0)
    assert rep.accesses > 10**7


def test_block_restricted_shapes():
    rep = check("prefix", batch=8, seqlen=512, D=256, dtype="f32", out=False, chunk=0)
    assert rep.launches == 2  # chunked: chunk pass + carry
    check("scan", batch=8, seqlen=32, D=256, dtype="f32", res="x", chunk=0)
    check("commit", batch=8, seqlen=32, D=256, dtype="f32", out=False, chunk=0)


def test_ragged_serving_shapes():
    import synth
    lens = synth.ragged_block_lengths()
    check("scan", lengths=lens, D=4096, chunk=0)
    check("commit", lengths=lens, D=4096, out=False, chunk=0)


def test_ragged_prefix_shape():
    import synth
    rep = check("prefix", lengths=synth.ragged_prefix_lengths(), D=4096, out=False, chunk=0)
    assert rep.launches == 2 and rep.accesses > 10**8


# ---- the backward ---------------------------------------------------------------
def make_grad(a, heap, *, dtype="bf16", grads=("dx", "ddt", "dBm", "dCm", "dA", "dDskip", "dh_in",
                                               "ds"), dh_out=True, pad_row=0):
    """Gradient buffers for the forward call `a` (layout as its x)."""
    es = 2 if dtype == "bf16" else 4
    D, N = a.dim, 16
    tok = a.total_tokens if a.cu_seqlens else a.batch * a.seqlen
    g = _abi.GradArgs()

    def tensor():
        stride = D + pad_row
        if a.cu_seqlens:
            return heap.alloc(((tok - 1) * stride + D) * es if tok else 0), stride, 0
        bst = a.seqlen * stride
        ext = ((a.batch - 1) * bst + (a.seqlen - 1) * stride + D) if tok else 0
        return heap.alloc(ext * es), stride, 0

    g.dout, g.dout_stride, g.dout_batch_stride = tensor()
    if dh_out:
        g.dh_out = heap.alloc(4 * a.batch * D * N)
    for n in ("dx", "ddt"):
        if n in grads:
            p, st, bst = tensor()
            setattr(g, n, p)
            setattr(g, n + "_stride", st)
            setattr(g, n + "_batch_stride", bst)
    sizes = {"dBm": tok * N, "dCm": tok * N, "dA": D * N, "dDskip": D, "dh_in": a.batch * D * N,
             "ds": 1}
    for n, cnt in sizes.items():
        if n in grads and (n != "ds" or a.res):
            setattr(g, n, heap.alloc(4 * cnt))
    need = _abi.backward_workspace_size(a, g)
    if need:
        g.workspace, g.workspace_bytes = heap.alloc(need), need
    return g


def check_bwd(grads=None, dh_out=True, reverse=True, **kw):
    res = kw.pop("res", "none")
    a, cu = make_args("scan", res=res, **kw)
    heap = FakeHeap()
    heap.next = BASE + (1 << 40)   # away from the forward buffers
    g = make_grad(a, heap, dtype=kw.get("dtype", "bf16"), dh_out=dh_out,
                  pad_row=kw.get("pad_row", 0),
                  **({"grads": grads} if grads is not None else {}))
    st, rep = _abi.check_access_backward(a, g, cu, reverse=reverse)
    msg = rep.message.decode() or _abi.last_error()
    assert st == _abi.R2L_OK, "backward %s: %s" % (kw, msg)
    return rep


BWD_EDGE = [
    dict(lengths=[0, 0]),
    dict(lengths=[5, 0, 1, 7, 8, 9, 64, 65, 130]),
    dict(batch=3, seqlen=0),
    dict(batch=2, seqlen=1),
    dict(batch=2, seqlen=73, D=37),
    dict(batch=2, seqlen=200, D=100, pad_row=8, pad_batch=40),
    dict(lengths=[300, 17], D=1),
]


@pytest.mark.parametrize("case", range(len(BWD_EDGE)))
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_edge_cases(case, dtype):
    kw = dict(BWD_EDGE[case], dtype=dtype)
    kw.setdefault("D", 64)
    for res in ("none", "x", "sep"):
        check_bwd(res=res, h_in=True, **kw)
        check_bwd(res=res, h_in=True, reverse=False, **kw)
    check_bwd(grads=("dx",), dh_out=False, **kw)
    check_bwd(grads=("dBm", "dA"), **kw)
    check_bwd(grads=(), **kw)


def test_backward_workspace_tracks_the_outputs():
    a, _ = make_args("scan", batch=4, seqlen=100, D=64)
    heap = FakeHeap()
    heap.next = BASE + (1 << 40)
    full = _abi.backward_workspace_size(a, make_grad(a, heap))
    only_dx = _abi.backward_workspace_size(a, make_grad(a, heap, grads=("dx",)))
    assert full > only_dx > 0   # checkpoints always; partial sums only when wanted


BWD_CHUNKED = [
    dict(lengths=[5, 0, 1, 64, 65, 130, 300], chunk=16),
    dict(lengths=[5, 0, 1, 64, 65, 130, 300], chunk=13),    # rounded up to 16
    dict(lengths=[7, 8, 9, 41], chunk=8),
    dict(batch=2, seqlen=200, D=37, chunk=40),
    dict(batch=2, seqlen=200, D=100, pad_row=8, pad_batch=40, chunk=64),
    dict(batch=2, seqlen=1000, D=64, chunk=0),                # chunked by the planner
]


@pytest.mark.parametrize("case", range(len(BWD_CHUNKED)))
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_backward_chunked_state_pass(case, dtype):
    """Phase 1 cut into chunks scanned from zero, the carry of the chunk entry
    states, and phase 2 reading them beside the chunk-local checkpoints."""
    kw = dict(BWD_CHUNKED[case], dtype=dtype)
    kw.setdefault("D", 64)
    for res in ("none", "x"):
        for reverse in (True, False):
            rep = check_bwd(res=res, h_in=True, reverse=reverse, **kw)
            assert rep.launches == 4   # phase 1, carry, phase 2, the sums
    check_bwd(grads=("dx",), dh_out=False, **kw)


def test_backward_chunk_plan():
    """The planner chunks phase 1 only when there are too few channels, in
    whole checkpoint groups; chunk_tokens < 0 keeps it whole."""
    heap = FakeHeap()
    heap.next = BASE + (1 << 40)
    a, _ = make_args("scan", batch=2, seqlen=1000, D=64, chunk=0)
    g = make_grad(a, heap)
    chunked = _abi.backward_workspace_size(a, g)
    a.chunk_tokens = -1
    assert chunked > _abi.backward_workspace_size(a, g)
    a, _ = make_args("scan", batch=64, seqlen=32, D=2048, chunk=0)
    g = make_grad(a, heap)
    auto = _abi.backward_workspace_size(a, g)
    a.chunk_tokens = -1
    assert auto == _abi.backward_workspace_size(a, g)


def test_backward_benchmarked_shapes():
    rep = check_bwd(batch=64, seqlen=32, D=2048, res="x", chunk=0)
    assert rep.launches == 3   # phase 1, phase 2, the sums: 131072 channels need no chunks
    rep = check_bwd(batch=8, seqlen=4096, D=4096, chunk=0)
    assert rep.launches == 4   # phase 1 in chunks, the carry, phase 2, the sums


# ---- the saving forward and the backward from its checkpoints -------------------------
def check_save(reverse=True, **kw):
    """Replay r2l_scan_save (prefix_scan_save) and then the backward from its
    checkpoints."""
    res = kw.pop("res", "none")
    a, cu = make_args("scan", res=res, **kw)
    # the saving forward plans its own workspace (chunks in whole groups of 8 tokens)
    need = _abi.workspace_size(_abi.R2L_OP_SAVE if reverse else _abi.R2L_OP_PREFIX_SAVE, a)
    heap = FakeHeap()
    heap.next = BASE + (1 << 40)
    a.workspace, a.workspace_bytes = (heap.alloc(need), need) if need else (None, 0)
    if not reverse and not a.out and not a.h_out:   # prefix_scan_state needs out or h_out
        a.h_out = heap.alloc(4 * a.batch * a.dim * 16)
    nbytes = _abi.checkpoint_size(a)
    ckpt = heap.alloc(nbytes)
    st, rep = _abi.check_access_save(a, ckpt, nbytes, cu, reverse=reverse)
    msg = rep.message.decode() or _abi.last_error()
    assert st == _abi.R2L_OK, "save %s: %s" % (kw, msg)
    heap.next = BASE + (2 << 40)
    g = make_grad(a, heap, dtype=kw.get("dtype", "bf16"), pad_row=kw.get("pad_row", 0))
    st, brep = _abi.check_access_backward_saved(a, g, ckpt, nbytes, cu, reverse=reverse)
    msg = brep.message.decode() or _abi.last_error()
    assert st == _abi.R2L_OK, "backward from checkpoints %s: %s" % (kw, msg)
    return a, rep, brep


SAVE_EDGE = BWD_EDGE + BWD_CHUNKED + [
    dict(lengths=[700, 1, 0, 333, 64, 1025], D=96, chunk=100),   # rounded up to 104
    dict(batch=2, seqlen=300, D=256, chunk=64, pad_row=8, pad_batch=40),
]


@pytest.mark.parametrize("reverse", [True, False], ids=["r2l", "l2r"])
@pytest.mark.parametrize("case", range(len(SAVE_EDGE)))
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_save_and_saved_backward(case, dtype, reverse):
    """Every checkpoint row the backward reads is written by the saving
    forward (the replay checks it), and neither call leaves its buffers."""
    kw = dict(SAVE_EDGE[case], dtype=dtype)
    kw.setdefault("D", 64)
    for res in ("none", "x", "sep", "inplace"):
        for h in (False, True):
            check_save(res=res, h_in=h, h_out=h, reverse=reverse, **kw)
    check_save(res="x", s=0.0, reverse=reverse, **kw)   # gate closed: a state-only scan stores them
    # gate closed, out = x with a separate residual: the state-only scan that
    # stores them reads x before the residual copy overwrites it
    check_save(res="sep_into_x", s=0.0, h_out=True, reverse=reverse, **kw)


def test_save_plans():
    """Unchunked, the saving forward runs r2l_scan's launches; the backward
    from its checkpoints runs no forward state pass; the checkpoint rows
    follow the documented count."""
    a, rep, brep = check_save(batch=64, seqlen=32, D=2048, res="x", chunk=0)
    assert rep.launches == 1 and brep.launches == 2
    assert _abi.checkpoint_size(a) == (64 * 32 // 8 + 64 + 1) * 2048 * 16 * 4
    a, rep, brep = check_save(batch=8, seqlen=4096, D=4096, chunk=0)
    assert rep.launches == 3 and brep.launches == 2       # chunk states, carry, readout
    a, rep, brep = check_save(batch=2, seqlen=64, D=64, res="x", s=0.0)
    assert rep.launches == 2                              # res copied to out, state-only scan
    a, rep, brep = check_save(batch=2, seqlen=64, D=64, res="inplace", s=0.0)
    assert rep.launches == 1                              # out is res: the state-only scan
    a, rep, brep = check_save(batch=2, seqlen=64, D=64, res="sep_into_x", s=0.0, h_out=True)
    assert rep.launches == 3                              # state scan (h_out), checkpoints, copy
    a, rep, brep = check_save(lengths=[0, 0], D=64)
    assert _abi.checkpoint_size(a) == 0 or rep.launches <= 1


def test_save_rejects_bad_arguments():
    a, cu = make_args("scan", batch=2, seqlen=64, D=64, res="x")
    nbytes = _abi.checkpoint_size(a)
    heap = FakeHeap()
    heap.next = BASE + (1 << 40)
    ckpt = heap.alloc(nbytes)
    st, _ = _abi.check_access_save(a, ckpt, nbytes - 4, cu)
    assert st == _abi.R2L_ERR_WORKSPACE
    st, _ = _abi.check_access_save(a, None, nbytes, cu)
    assert st == _abi.R2L_ERR_INVALID_ARG
    st, _ = _abi.check_access_save(a, ckpt + 4, nbytes, cu)
    assert st == _abi.R2L_ERR_MISALIGNED
    st, _ = _abi.check_access_save(a, a.x, nbytes, cu)     # overlaps x
    assert st == _abi.R2L_ERR_ALIAS
    a.state_split = 2
    st, _ = _abi.check_access_save(a, ckpt, nbytes, cu)
    assert st == _abi.R2L_ERR_UNSUPPORTED
    a.state_split = 0
    g = make_grad(a, heap)
    st, _ = _abi.check_access_backward_saved(a, g, ckpt, nbytes - 4, cu)
    assert st == _abi.R2L_ERR_WORKSPACE
    st, _ = _abi.check_access_backward_saved(a, g, g.dx, nbytes, cu)    # overlaps dx
    assert st == _abi.R2L_ERR_ALIAS


# ---- the bidirectional scan ---------------------------------------------------------
def make_dir(a, heap, kind, *, dtype="bf16", pad_row=0, bc_shift=0):
    """Reverse-direction parameters for the forward call `a`: "shared" (NULL
    struct), "separate" (every tensor its own) or "partial" (dt and A only)."""
    if kind == "shared":
        return None
    es = 2 if dtype == "bf16" else 4
    D, N = a.dim, 16
    tok = a.total_tokens if a.cu_seqlens else a.batch * a.seqlen

    def tensor(cols, lead=0):
        stride = cols + pad_row
        if a.cu_seqlens:
            p = heap.alloc(((tok - 1) * stride + cols + lead) * es if tok else 0)
        else:
            ext = ((a.batch - 1) * a.seqlen * stride + (a.seqlen - 1) * stride + cols + lead) \
                if tok else 0
            p = heap.alloc(ext * es)
        return (p + lead * es if p is not None else None), stride, 0

    r = _abi.DirArgs()
    r.dt, r.dt_stride, r.dt_batch_stride = tensor(D)
    r.A = heap.alloc(4 * D * N)
    if kind == "separate":
        r.Bm, r.Bm_stride, r.Bm_batch_stride = tensor(N, bc_shift)
        r.Cm, r.Cm_stride, r.Cm_batch_stride = tensor(N, bc_shift)
        r.Dskip = heap.alloc(4 * D)
    return r


def check_bidir(rev="separate", **kw):
    a, cu = make_args("scan", **kw)
    heap = FakeHeap()
    heap.next = BASE + (1 << 40)   # away from the forward buffers
    a.workspace, a.workspace_bytes = None, 0
    r = make_dir(a, heap, rev, dtype=kw.get("dtype", "bf16"), pad_row=kw.get("pad_row", 0),
                 bc_shift=kw.get("bc_shift", 0))
    need = _abi.workspace_size(_abi.R2L_OP_BIDIR, a)
    if need:
        a.workspace, a.workspace_bytes = heap.alloc(need), need
    st, rep = _abi.check_access_bidir(a, r, cu)
    msg = rep.message.decode() or _abi.last_error()
    assert st == _abi.R2L_OK, "bidir %s %s: %s" % (rev, kw, msg)
    return rep


@pytest.mark.parametrize("case", range(len(EDGE)))
@pytest.mark.parametrize("rev", ["shared", "separate", "partial"])
def test_bidir_edge_cases(case, rev):
    kw = dict(EDGE[case])
    for res in ("none", "x", "sep", "inplace"):
        for dtype in ("bf16", "f32"):
            check_bidir(rev, res=res, dtype=dtype, **kw)
    check_bidir(rev, res="x", s=0.0, **kw)     # gate closed: copy (+ forward state)
    check_bidir(rev, res="x", bc_shift=1, **kw)


def test_bidir_plans():
    # unchunked: one fused launch; the workspace holds the fp32 reverse rows
    rep = check_bidir(batch=64, seqlen=32, D=2048, res="x", chunk=0)
    assert rep.launches == 1 and rep.vector_staging == 2
    a, _ = make_args("scan", batch=64, seqlen=32, D=2048, res="x", chunk=0)
    assert _abi.workspace_size(_abi.R2L_OP_BIDIR, a) == 64 * 32 * 2048 * 4
    # chunked: the reverse plan (chunk pass, carry, readout pass), then the forward one
    rep = check_bidir(batch=2, seqlen=900, D=64, chunk=100, h_in=True, h_out=True)
    assert rep.launches == 6
    rep = check_bidir(batch=8, seqlen=4096, D=4096, chunk=0)
    assert rep.launches == 6 and rep.accesses > 10**7
    # gate closed: the residual copied, the forward state scanned when wanted
    assert check_bidir(batch=3, seqlen=40, D=64, res="x", s=0.0).launches == 1
    assert check_bidir(batch=3, seqlen=40, D=64, res="x", s=0.0, h_out=True).launches == 2
    assert check_bidir(batch=3, seqlen=40, D=64, res="inplace", s=0.0).launches == 0


def test_bidir_random_plans():
    rng = random.Random(4321)
    for _ in range(150):
        kw = dict(dtype=rng.choice(["bf16", "f32"]), D=rng.choice([1, 5, 64, 100, 256, 513]),
                  chunk=rng.choice([-1, 0, 16, 33, 64, 200]), h_in=rng.random() < 0.5,
                  h_out=rng.random() < 0.5, pad_row=rng.choice([0, 0, 1, 8]),
                  bc_shift=rng.choice([0, 0, 1]), res=rng.choice(["none", "x", "sep", "inplace"]),
                  s=rng.choice([0.05, 0.05, 0.0]))
        if rng.random() < 0.5:
            kw["lengths"] = [rng.choice([0, 1, 2, 31, 64, 65, 130, 300]) for _ in range(rng.randint(1, 6))]
        else:
            kw.update(batch=rng.randint(1, 5), seqlen=rng.choice([0, 1, 8, 63, 64, 65, 257]),
                      pad_batch=rng.choice([0, 0, 24]))
        check_bidir(rng.choice(["shared", "separate", "partial"]), **kw)


def test_bidir_rejects_bad_arguments():
    a, cu = make_args("scan", batch=2, seqlen=40, D=64, res="x")
    heap = FakeHeap()
    heap.next = BASE + (1 << 40)
    need = _abi.workspace_size(_abi.R2L_OP_BIDIR, a)
    a.workspace, a.workspace_bytes = heap.alloc(need), need
    r = make_dir(a, heap, "separate")
    assert _abi.check_access_bidir(a, r, cu)[0] == _abi.R2L_OK
    # the reverse dt overlapping out
    bad = _abi.DirArgs.from_buffer_copy(r)
    bad.dt = a.out
    assert _abi.check_access_bidir(a, bad, cu)[0] == _abi.R2L_ERR_ALIAS
    # too little workspace
    a.workspace_bytes = need - 4
    assert _abi.check_access_bidir(a, r, cu)[0] == _abi.R2L_ERR_WORKSPACE
    a.workspace_bytes = need
    # the workspace overlapping the reverse Bm
    bad = _abi.DirArgs.from_buffer_copy(r)
    bad.Bm = a.workspace
    assert _abi.check_access_bidir(a, bad, cu)[0] == _abi.R2L_ERR_ALIAS
    # several lanes per channel are not built for it
    a.state_split = 2
    assert _abi.check_access_bidir(a, r, cu)[0] == _abi.R2L_ERR_UNSUPPORTED


# ---- the sidecar block ---------------------------------------------------------------
def make_sidecar(*, dtype="bf16", dm=64, di=128, R=8, K=4, batch=None, seqlen=None, lengths=None,
                 s=0.5, in_place=False, pad_row=0, bias=True):
    es = 2 if dtype == "bf16" else 4
    N = 16
    heap = FakeHeap()
    a = _abi.SidecarArgs()
    a.gemm = heap.alloc(64)   # a GEMM context handle; the replay never looks inside it
    a.d_model, a.d_inner, a.dstate, a.dt_rank, a.d_conv = dm, di, N, R, K
    a.dtype = _abi.R2L_DTYPE_BF16 if dtype == "bf16" else _abi.R2L_DTYPE_F32
    cu = None
    if lengths is not None:
        a.batch = len(lengths)
        cu = [0] + [int(v) for v in np.cumsum(lengths)]
        a.total_tokens, a.max_seqlen = cu[-1], max(lengths) if lengths else 0
        a.cu_seqlens = heap.alloc(4 * (a.batch + 1))
        T = cu[-1]
    else:
        a.batch, a.seqlen = batch, seqlen
        T = batch * seqlen
    stride = dm + pad_row

    def rows(n, ld, cols):
        return heap.alloc(((n - 1) * ld + cols) * es if n else 0)

    a.hidden, a.hidden_stride = rows(T, stride, dm), stride
    a.out, a.out_stride = (a.hidden, stride) if in_place else (rows(T, stride, dm), stride)
    a.W_in = heap.alloc(2 * di * dm * es)
    a.conv_w = heap.alloc(4 * di * K)
    a.W_x = heap.alloc((R + 2 * N) * di * es)
    a.W_dt = heap.alloc(di * R * es)
    a.A = heap.alloc(4 * di * N)
    a.W_out = heap.alloc(dm * di * es)
    if bias:
        a.conv_b, a.dt_bias, a.Dskip = heap.alloc(4 * di), heap.alloc(4 * di), heap.alloc(4 * di)
    a.s = s
    need = _abi.sidecar_workspace_size(a)
    if need:
        a.workspace, a.workspace_bytes = heap.alloc(need), need
    return a, cu


def check_sidecar(**kw):
    a, cu = make_sidecar(**kw)
    st, rep = _abi.check_access_sidecar(a, cu)
    msg = rep.message.decode() or _abi.last_error()
    assert st == _abi.R2L_OK, "sidecar %s: %s" % (kw, msg)
    return rep


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_sidecar_plans(dtype):
    # six launches: 4 GEMMs, the conv, one scan launch (unchunked)
    rep = check_sidecar(dtype=dtype, batch=2, seqlen=40)
    assert rep.launches == 6
    # ragged edges, short and long sequences (the scan chunks: 8 launches)
    check_sidecar(dtype=dtype, lengths=[5, 0, 1, 64, 65, 130, 3])
    rep = check_sidecar(dtype=dtype, lengths=[2000, 1, 700], di=64)
    assert rep.launches == 8
    check_sidecar(dtype=dtype, batch=3, seqlen=33, K=1, R=16, bias=False, pad_row=8)
    check_sidecar(dtype=dtype, batch=1, seqlen=7, K=2, in_place=True)
    # s = 0: a copy of hidden, or nothing in place
    assert check_sidecar(dtype=dtype, batch=2, seqlen=9, s=0.0).launches == 1
    assert check_sidecar(dtype=dtype, batch=2, seqlen=9, s=0.0, in_place=True).launches == 0
    assert check_sidecar(dtype=dtype, lengths=[0, 0]).launches == 0


def test_sidecar_benchmarked_shape():
    rep = check_sidecar(batch=64, seqlen=32, dm=2048, di=4096, R=128)
    assert rep.launches == 6 and rep.vector_staging == 1


def test_sidecar_projection_shapes():
    """d_inner off the conv's channel tiles, dt_rank 8 to 232, ragged sequences,
    conv chunks with tails."""
    for kw in (dict(lengths=[31, 0, 1, 33, 64, 97], di=136, R=8),
               dict(batch=3, seqlen=45, di=520, R=24, K=3),
               dict(lengths=[5, 300, 2], di=1032, R=224, pad_row=8),
               dict(batch=2, seqlen=70, di=512, R=96, K=1, bias=False),
               dict(batch=2, seqlen=20, R=232)):
        assert check_sidecar(**kw).launches == 6


def test_sidecar_rejects_bad_arguments():
    a, cu = make_sidecar(batch=2, seqlen=16)
    assert _abi.check_access_sidecar(a, cu)[0] == _abi.R2L_OK
    bad = _abi.SidecarArgs.from_buffer_copy(a)
    bad.d_conv = 5
    assert _abi.check_access_sidecar(bad, cu)[0] == _abi.R2L_ERR_UNSUPPORTED
    bad = _abi.SidecarArgs.from_buffer_copy(a)
    bad.d_inner = 100
    assert _abi.check_access_sidecar(bad, cu)[0] == _abi.R2L_ERR_UNSUPPORTED
    bad = _abi.SidecarArgs.from_buffer_copy(a)
    bad.workspace_bytes -= 256
    assert _abi.check_access_sidecar(bad, cu)[0] == _abi.R2L_ERR_WORKSPACE
    bad = _abi.SidecarArgs.from_buffer_copy(a)
    bad.out = bad.W_in            # the output over a weight
    assert _abi.check_access_sidecar(bad, cu)[0] == _abi.R2L_ERR_ALIAS
    bad = _abi.SidecarArgs.from_buffer_copy(a)
    bad.hidden_stride = 65        # rows off 16-byte boundaries
    assert _abi.check_access_sidecar(bad, cu)[0] == _abi.R2L_ERR_MISALIGNED
    bad = _abi.SidecarArgs.from_buffer_copy(a)
    bad.dt_rank = 3
    assert _abi.check_access_sidecar(bad, cu)[0] == _abi.R2L_ERR_UNSUPPORTED
    bad = _abi.SidecarArgs.from_buffer_copy(a)
    bad.W_x = None
    assert _abi.check_access_sidecar(bad, cu)[0] == _abi.R2L_ERR_INVALID_ARG
    bad = _abi.SidecarArgs.from_buffer_copy(a)
    bad.gemm = None               # s != 0 needs the caller's GEMM context
    assert _abi.check_access_sidecar(bad, cu)[0] == _abi.R2L_ERR_INVALID_ARG
    assert "gemm" in _abi.last_error()
