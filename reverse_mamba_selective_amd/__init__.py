"""MI355X-native R2L / forward selective scans (the hot path of the Bifocal dLLM /
R2LM method and of block-diffusion Mamba prefix caching).

Thin PyTorch-facing binding over the C ABI in ``include/r2l_scan.h``: it only
checks tensor layouts, fills the argument struct and passes torch's current
HIP stream. Every step of the computation runs in the library's gfx950
kernels; torch provides device memory and streams. The first call fails
(ImportError) when ``libr2l_scan.so`` is not built: there is no fallback.

Tensor layouts
    x, dt, res, out   [batch, L, D] (dense) or [tokens, D] (ragged, with cu_seqlens)
    Bm, Cm            [batch, L, N] or [tokens, N]
    A                 [D, N] fp32;  Dskip [D] fp32
    h_in, h_out       [batch, D, N] fp32
The last dimension must be contiguous and the token rows evenly strided.
x, dt, Bm, Cm, res and out share one dtype: float32 or bfloat16.
"""
from __future__ import annotations

import torch

from . import _abi
from ._abi import R2LError  # noqa: F401

__all__ = ["r2l_scan", "r2l_scan_noalloc", "GemmContext", "prefix_scan_state", "block_commit_state", "bidir_scan", "sidecar_forward",
           "sidecar_tune",
           "bind_sidecar", "SIDECAR_WEIGHTS",
           "workspace_size", "bind",
           "BoundCall", "R2LError", "library_path", "r2l_scan_backward", "prefix_scan_backward",
           "bind_backward",
           "BoundBackward", "R2LScan", "GRADS", "r2l_scan_save", "prefix_scan_save",
           "checkpoint_size"]

_DTYPES = {torch.float32: _abi.R2L_DTYPE_F32, torch.bfloat16: _abi.R2L_DTYPE_BF16}


def library_path() -> str:
    return _abi.LIB_PATH


def _rows(t, cols, name):
    """(pointer, token stride, batch stride, rows) of a [batch, L, cols] or
    [tokens, cols] view; strides in elements."""
    if t is None:
        return None, 0, 0, 0
    if t.dim() not in (2, 3) or t.shape[-1] != cols:
        raise ValueError("%s must be [batch, L, %d] or [tokens, %d], got %s"
                         % (name, cols, cols, tuple(t.shape)))
    if t.shape[-1] > 1 and t.stride(-1) != 1:
        raise ValueError("%s: last dimension must be contiguous" % name)
    if any(st < 0 for st in t.stride()):
        raise ValueError("%s: negative strides are not supported" % name)
    rs = max(int(t.stride(-2)), cols)
    if t.dim() == 3:
        return t.data_ptr(), rs, int(t.stride(0)), int(t.shape[0] * t.shape[1])
    return t.data_ptr(), rs, 0, int(t.shape[0])


def _ptr(t):
    return None if t is None else t.data_ptr()


def _check_f32(t, shape, name):
    if t is None:
        return
    if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError("%s must be a contiguous float32 tensor of shape %s, got %s %s"
                         % (name, tuple(shape), t.dtype, tuple(t.shape)))


def _fill(x, dt, Bm, Cm, A, Dskip, cu_seqlens, max_seqlen, h_in, h_out, res, s, out,
          delta_softplus, chunk_tokens, state_split):
    if x.dtype not in _DTYPES:
        raise ValueError("x must be float32 or bfloat16, got %s" % x.dtype)
    for t, n in ((dt, "dt"), (Bm, "Bm"), (Cm, "Cm"), (res, "res"), (out, "out")):
        if t is not None and t.dtype != x.dtype:
            raise ValueError("%s has dtype %s but x has %s" % (n, t.dtype, x.dtype))
    D = int(x.shape[-1])
    if A.dim() != 2 or A.shape[0] != D:
        raise ValueError("A must be [D, N] with D = %d" % D)
    N = int(A.shape[1])
    a = _abi.ScanArgs()
    if cu_seqlens is not None:
        if x.dim() != 2:
            raise ValueError("ragged layout takes [tokens, D] tensors")
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
            raise ValueError("cu_seqlens must be a 1-D int32 tensor")
        batch = int(cu_seqlens.shape[0]) - 1
        if max_seqlen is None:
            max_seqlen = int((cu_seqlens[1:] - cu_seqlens[:-1]).max().item()) if batch > 0 else 0
        a.cu_seqlens = cu_seqlens.data_ptr()
        a.total_tokens = int(x.shape[0])
        a.max_seqlen = int(max_seqlen)
        a.batch = batch
    elif x.dim() == 3:
        a.batch, a.seqlen = int(x.shape[0]), int(x.shape[1])
    else:
        a.batch, a.seqlen = 1, int(x.shape[0])
    a.dim, a.dstate, a.dtype = D, N, _DTYPES[x.dtype]
    a.x, a.x_stride, a.x_batch_stride, rows = _rows(x, D, "x")
    for t, n, cols in ((dt, "dt", D), (Bm, "Bm", N), (Cm, "Cm", N), (res, "res", D),
                       (out, "out", D)):
        if t is None:
            continue
        if t.dim() != x.dim() or (t.dim() == 3 and t.shape[:2] != x.shape[:2]):
            raise ValueError("%s has shape %s, x has %s" % (n, tuple(t.shape), tuple(x.shape)))
        p, st, bst, r = _rows(t, cols, n)
        if r != rows:
            raise ValueError("%s has %d token rows, x has %d" % (n, r, rows))
        setattr(a, n, p)
        setattr(a, n + "_stride", st)
        setattr(a, n + "_batch_stride", bst)
    _check_f32(A, (D, N), "A")
    _check_f32(Dskip, (D,), "Dskip")
    _check_f32(h_in, (a.batch, D, N), "h_in")
    _check_f32(h_out, (a.batch, D, N), "h_out")
    a.A, a.Dskip = A.data_ptr(), _ptr(Dskip)
    a.h_in, a.h_out = _ptr(h_in), _ptr(h_out)
    a.s = float(s)
    a.delta_softplus = 1 if delta_softplus else 0
    a.chunk_tokens, a.state_split = int(chunk_tokens), int(state_split)
    return a


def _attach_workspace(op, a, workspace, device):
    need = _abi.workspace_size(op, a)
    if need:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=device)
        elif workspace.numel() * workspace.element_size() < need:
            raise ValueError("workspace has %d bytes, the plan needs %d"
                             % (workspace.numel() * workspace.element_size(), need))
        a.workspace, a.workspace_bytes = workspace.data_ptr(), need
    return workspace


def _run(func, op, a, workspace, device):
    workspace = _attach_workspace(op, a, workspace, device)
    with torch.cuda.device(device):
        stream = torch.cuda.current_stream(device).cuda_stream
    _abi.call(func, a, stream)


class BoundCall:
    """One entry-point call with its argument struct filled once.

    ``launch()`` queues it again on torch's current stream of the tensors'
    device (or on ``stream``, a raw hipStream_t). The tensors given to ``bind``
    (and the workspace) are kept alive by this object; their contents may
    change between launches, their storage may not.
    """

    def __init__(self, func, op, args, keep, workspace, device, rev=None, ckpt=None):
        self.func, self.op, self.args = func, op, args
        self._keep, self.workspace, self.device = keep, workspace, device
        self._fn = getattr(_abi.load(), func)
        self._ref = _abi.ctypes.byref(args)
        # bidir_scan takes the reverse direction's struct (or NULL) as well,
        # r2l_scan_save the checkpoint buffer and its size
        self.rev, self.ckpt = rev, ckpt
        if func == "bidir_scan":
            self._refs = (self._ref, _abi._dir_ref(rev))
        elif func in ("r2l_scan_save", "prefix_scan_save"):
            self._refs = (self._ref, _abi._fptr(ckpt.data_ptr()), ckpt.numel() * 4)
        else:
            self._refs = (self._ref,)

    def plan(self) -> dict:
        """The plan the library picks for this call (lanes per channel, chunking,
        workspace bytes, launches)."""
        return _abi.describe_plan(self.op, self.args)

    def launch(self, stream=None):
        """Queue the call on ``stream`` (a raw hipStream_t handle) or, when None,
        on torch's current stream of the device."""
        if stream is None:
            stream = torch.cuda.current_stream(self.device).cuda_stream
        st = self._fn(*self._refs, _abi._vp(stream))
        if st != _abi.R2L_OK:
            raise R2LError(st, self.func, _abi.last_error())


def bind(op: str, **kw) -> BoundCall:
    """Check and marshal the arguments of ``r2l_scan``, ``prefix_scan_state``,
    ``block_commit_state``, ``bidir_scan`` or ``r2l_scan_save`` once (same
    keywords as those functions; outputs must be given; the checkpoints of
    ``r2l_scan_save`` are allocated here unless ``ckpt`` is given, and are the
    returned object's ``ckpt``) and return a :class:`BoundCall`.
    """
    kw = dict(kw)
    ws = kw.pop("workspace", None)
    rev = kw.pop("rev", None)
    ckpt = kw.pop("ckpt", None)
    if rev is not None and op != "bidir_scan":
        raise ValueError("rev is an argument of bidir_scan only")
    if ckpt is not None and op not in ("r2l_scan_save", "prefix_scan_save"):
        raise ValueError("ckpt is an argument of r2l_scan_save and prefix_scan_save only")
    if op == "r2l_scan_save":
        func, code = "r2l_scan_save", _abi.R2L_OP_SAVE
        kw["state_split"] = 1
    elif op == "prefix_scan_save":
        func, code = "prefix_scan_save", _abi.R2L_OP_PREFIX_SAVE
        kw["state_split"] = 1
    elif op == "bidir_scan":
        func, code = "bidir_scan", _abi.R2L_OP_BIDIR
    elif op == "r2l_scan":
        func, code = "r2l_scan", _abi.R2L_OP_SCAN
    elif op == "prefix_scan_state":
        func, code = "prefix_scan_state", _abi.R2L_OP_PREFIX
    elif op == "block_commit_state":
        func, code = "block_commit_state", _abi.R2L_OP_COMMIT
        kw["h_out"] = kw.pop("state")
    else:
        raise ValueError("unknown entry point %r" % op)
    x = kw["x"]
    if op in ("r2l_scan", "bidir_scan", "r2l_scan_save", "prefix_scan_save") and \
            kw.get("out") is None:
        raise ValueError("bind() needs the output tensor")
    names = ("x", "dt", "Bm", "Cm", "A", "Dskip", "cu_seqlens", "max_seqlen", "h_in", "h_out",
             "res", "s", "out", "delta_softplus", "chunk_tokens", "state_split")
    defaults = {"Cm": None, "Dskip": None, "cu_seqlens": None, "max_seqlen": None,
                "h_in": None, "h_out": None, "res": None, "s": 0.0, "out": None,
                "delta_softplus": True, "chunk_tokens": 0, "state_split": 0}
    unknown = set(kw) - set(names)
    if unknown:
        raise ValueError("unknown arguments %s" % sorted(unknown))
    vals = [kw.get(n, defaults.get(n)) for n in names]
    a = _fill(*vals)
    r = _fill_dir(a, x, rev) if op == "bidir_scan" else None
    ws = _attach_workspace(code, a, ws, x.device)
    keep = [v for v in vals if isinstance(v, torch.Tensor)] + list((rev or {}).values())
    if op in ("r2l_scan_save", "prefix_scan_save"):
        ckpt = _checkpoints(a, ckpt, x.device)
    return BoundCall(func, code, a, keep, ws, x.device, rev=r, ckpt=ckpt)


def _checkpoints(a, ckpt, device):
    need = _abi.checkpoint_size(a)
    if ckpt is None:
        return torch.empty(max(need // 4, 1), dtype=torch.float32, device=device)
    if ckpt.dtype != torch.float32 or not ckpt.is_contiguous() or ckpt.numel() * 4 < need:
        raise ValueError("ckpt must be a contiguous fp32 tensor of at least %d bytes" % need)
    return ckpt


def workspace_size(op: str, x, A, *, cu_seqlens=None, max_seqlen=None, out=True,
                   chunk_tokens=0, state_split=0) -> int:
    """Workspace bytes for op in {"r2l_scan", "prefix_scan_state", "block_commit_state",
    "bidir_scan", "r2l_scan_save", "prefix_scan_save"}."""
    codes = {"r2l_scan": _abi.R2L_OP_SCAN, "prefix_scan_state": _abi.R2L_OP_PREFIX,
             "block_commit_state": _abi.R2L_OP_COMMIT, "bidir_scan": _abi.R2L_OP_BIDIR,
             "r2l_scan_save": _abi.R2L_OP_SAVE, "prefix_scan_save": _abi.R2L_OP_PREFIX_SAVE}
    a = _fill(x, None, None, None, A, None, cu_seqlens, max_seqlen, None, None, None, 0.0,
              None, True, chunk_tokens, state_split)
    if out:
        a.out = 1  # only "is a readout requested" is read
    return _abi.workspace_size(codes[op], a)


def r2l_scan(x, dt, Bm, Cm, A, Dskip=None, *, cu_seqlens=None, max_seqlen=None, h_in=None,
             h_out=None, res=None, s=0.0, out=None, delta_softplus=True, chunk_tokens=0,
             state_split=0, workspace=None):
    """The R2L stream: reverse selective scan with readout and gated residual.

    out[t] = y_t (res None) or res[t] + s*y_t (s == 0: res[t] bit for bit). ``out``
    may be ``x`` or ``res`` itself (in-place hook update). ``h_out`` receives the
    state after the leftmost token. Returns ``out``.
    """
    if out is None:
        out = torch.empty_like(x)
    a = _fill(x, dt, Bm, Cm, A, Dskip, cu_seqlens, max_seqlen, h_in, h_out, res, s, out,
              delta_softplus, chunk_tokens, state_split)
    _run("r2l_scan", _abi.R2L_OP_SCAN, a, workspace, x.device)
    return out


def r2l_scan_noalloc(x, dt, Bm, Cm, A, Dskip=None, *, out, cu_seqlens=None, max_seqlen=None,
                     h_in=None, h_out=None, res=None, s=0.0, delta_softplus=True,
                     chunk_tokens=0, state_split=0):
    """``r2l_scan`` that allocates nothing, for callers that cannot (graph
    capture, serving loops): ``out`` must be given, and a chunked plan's carry
    data goes to the library's own device scratch array (``NOALLOC_SCRATCH_BYTES``
    per GPU); a plan needing more raises. Calls that may overlap on one GPU
    (other streams or threads) race on that array. Returns ``out``."""
    a = _fill(x, dt, Bm, Cm, A, Dskip, cu_seqlens, max_seqlen, h_in, h_out, res, s, out,
              delta_softplus, chunk_tokens, state_split)
    stream = torch.cuda.current_stream(x.device).cuda_stream
    _abi.call("r2l_scan_noalloc", a, stream)
    return out


NOALLOC_SCRATCH_BYTES = _abi.NOALLOC_SCRATCH_BYTES


def checkpoint_size(x, A, *, cu_seqlens=None, max_seqlen=None) -> int:
    """Bytes of the checkpoints that ``r2l_scan_save`` stores for this shape."""
    a = _fill(x, None, None, None, A, None, cu_seqlens, max_seqlen, None, None, None, 0.0, None,
              True, 0, 0)
    return _abi.checkpoint_size(a)


def r2l_scan_save(x, dt, Bm, Cm, A, Dskip=None, *, cu_seqlens=None, max_seqlen=None,
                  h_in=None, h_out=None, res=None, s=0.0, out=None, delta_softplus=True,
                  chunk_tokens=0, ckpt=None, workspace=None, _reverse=True):
    """``r2l_scan`` that also stores the states the backward needs (the state
    entering every 8th visited position of each sequence). Returns (out, ckpt);
    ckpt is an fp32 tensor to hand to ``r2l_scan_backward(..., ckpt=ckpt)``
    with the same forward arguments."""
    if out is None:
        out = torch.empty_like(x)
    a = _fill(x, dt, Bm, Cm, A, Dskip, cu_seqlens, max_seqlen, h_in, h_out, res, s, out,
              delta_softplus, chunk_tokens, 1)
    ckpt = _checkpoints(a, ckpt, x.device)
    op = _abi.R2L_OP_SAVE if _reverse else _abi.R2L_OP_PREFIX_SAVE
    workspace = _attach_workspace(op, a, workspace, x.device)
    with torch.cuda.device(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
    _abi.call_save(a, ckpt.data_ptr(), ckpt.numel() * 4, stream, reverse=_reverse)
    return out, ckpt


def prefix_scan_save(x, dt, Bm, Cm, A, Dskip=None, **kw):
    """The left-to-right stream (``prefix_scan_state`` with readout into
    ``out``) that also stores the backward's checkpoints; same keywords and
    result as ``r2l_scan_save``; hand ckpt to ``prefix_scan_backward``."""
    return r2l_scan_save(x, dt, Bm, Cm, A, Dskip, _reverse=False, **kw)


def prefix_scan_state(x, dt, Bm, A, *, cu_seqlens=None, max_seqlen=None, h_in=None,
                      h_out=None, Cm=None, Dskip=None, res=None, s=0.0, out=None,
                      delta_softplus=True, chunk_tokens=0, state_split=0, workspace=None):
    """Forward-only boundary state of each prefix (left to right from h_in).

    Returns h_out [batch, D, N] (allocated when not given). With ``Cm`` (and an
    optional ``out``) the forward readout is written too and (h_out, out) is
    returned.
    """
    batch = int(cu_seqlens.shape[0]) - 1 if cu_seqlens is not None else \
        (int(x.shape[0]) if x.dim() == 3 else 1)
    if h_out is None:
        h_out = torch.empty((batch, x.shape[-1], A.shape[1]), dtype=torch.float32,
                            device=x.device)
    if Cm is not None and out is None:
        out = torch.empty_like(x)
    a = _fill(x, dt, Bm, Cm, A, Dskip, cu_seqlens, max_seqlen, h_in, h_out, res, s, out,
              delta_softplus, chunk_tokens, state_split)
    _run("prefix_scan_state", _abi.R2L_OP_PREFIX, a, workspace, x.device)
    return (h_out, out) if Cm is not None else h_out


def block_commit_state(state, x, dt, Bm, A, *, cu_seqlens=None, max_seqlen=None, Cm=None,
                       Dskip=None, res=None, s=0.0, out=None, delta_softplus=True,
                       chunk_tokens=0, state_split=0, workspace=None):
    """Advance cached boundary states [batch, D, N] over committed blocks, in place.

    Returns ``state`` (and ``out`` when ``Cm`` asks for the block's forward readout).
    """
    if Cm is not None and out is None:
        out = torch.empty_like(x)
    a = _fill(x, dt, Bm, Cm, A, Dskip, cu_seqlens, max_seqlen, None, state, res, s, out,
              delta_softplus, chunk_tokens, state_split)
    _run("block_commit_state", _abi.R2L_OP_COMMIT, a, workspace, x.device)
    return (state, out) if Cm is not None else state


# ---- bidirectional scan -------------------------------------------------------
_DIR_KEYS = ("dt", "Bm", "Cm", "A", "Dskip")


def _fill_dir(a, x, rev):
    """``r2l_dir_args`` of the reverse direction from a dict with any of the
    keys dt, Bm, Cm, A, Dskip (a missing key shares the forward's tensor);
    None when nothing is given."""
    if not rev:
        return None
    unknown = set(rev) - set(_DIR_KEYS)
    if unknown:
        raise ValueError("unknown reverse-direction parameters %s" % sorted(unknown))
    D, N = int(a.dim), int(a.dstate)
    rows = _rows(x, D, "x")[3]
    r = _abi.DirArgs()
    for n, cols in (("dt", D), ("Bm", N), ("Cm", N)):
        t = rev.get(n)
        if t is None:
            continue
        if t.dtype != x.dtype:
            raise ValueError("reverse %s has dtype %s but x has %s" % (n, t.dtype, x.dtype))
        if t.dim() != x.dim() or (t.dim() == 3 and t.shape[:2] != x.shape[:2]):
            raise ValueError("reverse %s has shape %s, x has %s"
                             % (n, tuple(t.shape), tuple(x.shape)))
        p, st, bst, nr = _rows(t, cols, "reverse " + n)
        if nr != rows:
            raise ValueError("reverse %s has %d token rows, x has %d" % (n, nr, rows))
        setattr(r, n, p)
        setattr(r, n + "_stride", st)
        setattr(r, n + "_batch_stride", bst)
    _check_f32(rev.get("A"), (D, N), "reverse A")
    _check_f32(rev.get("Dskip"), (D,), "reverse Dskip")
    r.A, r.Dskip = _ptr(rev.get("A")), _ptr(rev.get("Dskip"))
    return r


def bidir_scan(x, dt, Bm, Cm, A, Dskip=None, *, rev=None, cu_seqlens=None, max_seqlen=None,
               h_in=None, h_out=None, res=None, s=0.0, out=None, delta_softplus=True,
               chunk_tokens=0, workspace=None):
    """Bidirectional full-window scan: the forward scan of x (dt, Bm, Cm, A,
    Dskip; from h_in) plus the reverse scan of x (``rev``: a dict with any of
    dt, Bm, Cm, A, Dskip, the rest shared; from zero), readouts added, then
    out = y (res None) or res + s*y (s == 0: res bit for bit). ``h_out``
    receives the forward direction's final state. Returns ``out``.
    """
    if out is None:
        out = torch.empty_like(x)
    a = _fill(x, dt, Bm, Cm, A, Dskip, cu_seqlens, max_seqlen, h_in, h_out, res, s, out,
              delta_softplus, chunk_tokens, 0)
    r = _fill_dir(a, x, rev)
    workspace = _attach_workspace(_abi.R2L_OP_BIDIR, a, workspace, x.device)
    with torch.cuda.device(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
    _abi.call_bidir(a, r, stream)
    return out


# ---- sidecar block --------------------------------------------------------------
SIDECAR_WEIGHTS = ("W_in", "conv_w", "conv_b", "W_x", "W_dt", "dt_bias", "A", "Dskip", "W_out")


class GemmContext:
    """A GEMM context of the library (r2l_gemm_context): one device's hipBLASLt
    handle and the algorithm chosen for each projection shape. Created on
    ``device`` (default: the current one); ``close()`` releases it (no call
    using it may still be queued). Pass it as ``gemm=`` to the sidecar calls;
    without one they use the device's default context, which this module
    creates on first use and keeps for the life of the process."""

    def __init__(self, device=None):
        self.device = torch.device("cuda", torch.cuda.current_device()) if device is None \
            else torch.device(device)
        with torch.cuda.device(self.device):
            self.handle = _abi.gemm_context_create()

    def close(self):
        if self.handle:
            with torch.cuda.device(self.device):
                _abi.gemm_context_destroy(self.handle)
            self.handle = 0

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


_default_gemm = {}


def default_gemm_context(device) -> GemmContext:
    """The device's default GEMM context (created on first use, never closed)."""
    idx = torch.device(device).index
    idx = torch.cuda.current_device() if idx is None else idx
    if idx not in _default_gemm:
        _default_gemm[idx] = GemmContext(torch.device("cuda", idx))
    return _default_gemm[idx]


def _fill_sidecar(hidden, w, s, cu_seqlens, max_seqlen, out, gemm=None):
    if hidden.dtype not in _DTYPES:
        raise ValueError("hidden must be float32 or bfloat16, got %s" % hidden.dtype)
    unknown = set(w) - set(SIDECAR_WEIGHTS)
    if unknown:
        raise ValueError("unknown sidecar weights %s" % sorted(unknown))
    for k in ("W_in", "conv_w", "W_x", "W_dt", "A", "W_out"):
        if w.get(k) is None:
            raise ValueError("the sidecar needs %s" % k)
    dm = int(hidden.shape[-1])
    di, N = int(w["A"].shape[0]), int(w["A"].shape[1])
    R, K = int(w["W_dt"].shape[1]), int(w["conv_w"].shape[1])
    a = _abi.SidecarArgs()
    if cu_seqlens is not None:
        if hidden.dim() != 2:
            raise ValueError("ragged layout takes [tokens, d_model] tensors")
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
            raise ValueError("cu_seqlens must be a 1-D int32 tensor")
        a.batch = int(cu_seqlens.shape[0]) - 1
        if max_seqlen is None:
            max_seqlen = int((cu_seqlens[1:] - cu_seqlens[:-1]).max().item()) if a.batch > 0 else 0
        a.cu_seqlens, a.total_tokens, a.max_seqlen = cu_seqlens.data_ptr(), int(hidden.shape[0]), \
            int(max_seqlen)
    elif hidden.dim() == 3:
        a.batch, a.seqlen = int(hidden.shape[0]), int(hidden.shape[1])
    else:
        a.batch, a.seqlen = 1, int(hidden.shape[0])
    a.d_model, a.d_inner, a.dstate, a.dt_rank, a.d_conv = dm, di, N, R, K
    a.dtype = _DTYPES[hidden.dtype]
    for t, n in ((hidden, "hidden"), (out, "out")):
        if t.dtype != hidden.dtype or tuple(t.shape) != tuple(hidden.shape):
            raise ValueError("%s must match hidden in shape and dtype" % n)
        if t.dim() == 3 and t.shape[0] > 1 and t.stride(0) != t.shape[1] * t.stride(1):
            raise ValueError("%s: the sequences' rows must be evenly strided" % n)
    a.hidden, a.hidden_stride = _rows(hidden, dm, "hidden")[:2]
    a.out, a.out_stride = _rows(out, dm, "out")[:2]
    shapes = {"W_in": (2 * di, dm), "W_x": (R + 2 * N, di), "W_dt": (di, R), "W_out": (dm, di)}
    for n, shape in shapes.items():
        t = w[n]
        if t.dtype != hidden.dtype or tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError("%s must be a contiguous %s tensor of shape %s" % (n, hidden.dtype, shape))
        setattr(a, n, t.data_ptr())
    for n, shape in (("conv_w", (di, K)), ("conv_b", (di,)), ("dt_bias", (di,)), ("A", (di, N)),
                     ("Dskip", (di,))):
        _check_f32(w.get(n), shape, n)
        setattr(a, n, _ptr(w.get(n)))
    a.s = float(s)
    if gemm is not None:
        a.gemm = gemm.handle
    elif a.s != 0.0 and hidden.is_cuda:
        a.gemm = default_gemm_context(hidden.device).handle
    return a


def _sidecar_workspace(a, workspace, device):
    need = _abi.sidecar_workspace_size(a)
    if need:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=device)
        elif workspace.numel() * workspace.element_size() < need:
            raise ValueError("workspace has %d bytes, the sidecar needs %d"
                             % (workspace.numel() * workspace.element_size(), need))
        a.workspace, a.workspace_bytes = workspace.data_ptr(), need
    return workspace


def sidecar_tune(hidden, weights: dict, *, s, cu_seqlens=None, max_seqlen=None, out=None,
                 workspace=None, gemm=None):
    """r2l_sidecar_tune for these arguments (see ``BoundSidecar.tune``)."""
    if out is None:
        out = torch.empty_like(hidden)
    a = _fill_sidecar(hidden, weights, s, cu_seqlens, max_seqlen, out, gemm)
    workspace = _sidecar_workspace(a, workspace, hidden.device)
    with torch.cuda.device(hidden.device):
        stream = torch.cuda.current_stream(hidden.device).cuda_stream
    _abi.call_sidecar(a, stream, tune=True)


def sidecar_forward(hidden, weights: dict, *, s, cu_seqlens=None, max_seqlen=None, out=None,
                    workspace=None, gemm=None):
    """The R2L sidecar block as a hook: out = hidden + s * sidecar(hidden)
    (in-projection, anti-causal depthwise conv + SiLU, x/dt projections, the
    R2L scan, SiLU(z) gate, out-projection; see r2l_sidecar_forward).
    ``weights``: W_in [2 di, dm], W_x [R + 2N, di], W_dt [di, R], W_out [dm, di]
    in hidden's dtype; conv_w [di, K], conv_b [di], dt_bias [di], A [di, N],
    Dskip [di] fp32 (conv_b, dt_bias, Dskip optional). ``out`` may be
    ``hidden``. ``gemm``: a :class:`GemmContext` (default: the device's).
    Returns ``out``."""
    if out is None:
        out = torch.empty_like(hidden)
    a = _fill_sidecar(hidden, weights, s, cu_seqlens, max_seqlen, out, gemm)
    workspace = _sidecar_workspace(a, workspace, hidden.device)
    with torch.cuda.device(hidden.device):
        stream = torch.cuda.current_stream(hidden.device).cuda_stream
    _abi.call_sidecar(a, stream)
    return out


class BoundSidecar:
    """One r2l_sidecar_forward call with its argument struct filled once."""

    def __init__(self, args, keep, workspace, device):
        self.args, self._keep, self.workspace, self.device = args, keep, workspace, device
        self._fn = _abi.load().r2l_sidecar_forward
        self._ref = _abi.ctypes.byref(args)

    def launch(self, stream=None):
        if stream is None:
            stream = torch.cuda.current_stream(self.device).cuda_stream
        st = self._fn(self._ref, _abi._vp(stream))
        if st != _abi.R2L_OK:
            raise R2LError(st, "r2l_sidecar_forward", _abi.last_error())

    def tune(self, stream=None):
        """Time the library's GEMM candidates for this call's shapes and keep the
        fastest (r2l_sidecar_tune; synchronizes the stream, overwrites the
        workspace)."""
        if stream is None:
            stream = torch.cuda.current_stream(self.device).cuda_stream
        _abi.call_sidecar(self.args, stream, tune=True)


def bind_sidecar(hidden, weights: dict, *, s, out, cu_seqlens=None, max_seqlen=None,
                 workspace=None, gemm=None) -> BoundSidecar:
    """Check and marshal a ``sidecar_forward`` call once (``out`` required)."""
    a = _fill_sidecar(hidden, weights, s, cu_seqlens, max_seqlen, out, gemm)
    workspace = _sidecar_workspace(a, workspace, hidden.device)
    keep = [hidden, out, cu_seqlens, gemm] + [v for v in weights.values() if v is not None]
    return BoundSidecar(a, keep, workspace, hidden.device)


# ---- backward ---------------------------------------------------------------
GRADS = ("dx", "ddt", "dBm", "dCm", "dA", "dDskip", "dh_in", "ds")


def _fill_grad(a, x, Bm, dout, dh_out, outs):
    g = _abi.GradArgs()
    D, N = int(a.dim), int(a.dstate)
    if dout.dtype != x.dtype or tuple(dout.shape) != tuple(x.shape):
        raise ValueError("dout must match x in shape and dtype")
    g.dout, g.dout_stride, g.dout_batch_stride, _ = _rows(dout, D, "dout")
    _check_f32(dh_out, (a.batch, D, N), "dh_out")
    g.dh_out = _ptr(dh_out)
    for n in ("dx", "ddt"):
        t = outs.get(n)
        if t is not None:
            if t.dtype != x.dtype or tuple(t.shape) != tuple(x.shape):
                raise ValueError("%s must match x in shape and dtype" % n)
            p, st, bst, _ = _rows(t, D, n)
            setattr(g, n, p)
            setattr(g, n + "_stride", st)
            setattr(g, n + "_batch_stride", bst)
    shapes = {"dBm": tuple(Bm.shape), "dCm": tuple(Bm.shape), "dA": (D, N), "dDskip": (D,),
              "dh_in": (a.batch, D, N), "ds": (1,)}
    for n, shape in shapes.items():
        _check_f32(outs.get(n), shape, n)
        setattr(g, n, _ptr(outs.get(n)))
    return g


class BoundBackward:
    """One r2l_scan_backward call with its argument structs filled once (see
    BoundCall); ``grads`` holds the output tensors."""

    def __init__(self, args, grad, keep, grads, workspace, device, reverse=True, ckpt=None):
        self.args, self.grad, self._keep = args, grad, keep
        self.grads, self.workspace, self.device = grads, workspace, device
        self.func = "r2l_scan_backward" if reverse else "prefix_scan_backward"
        self._a, self._g = _abi.ctypes.byref(args), _abi.ctypes.byref(grad)
        self._refs = (self._a, self._g)
        self.ckpt = ckpt
        if ckpt is not None:   # from the checkpoints of r2l_scan_save / prefix_scan_save
            self.func = self.func + "_saved"
            self._refs = (self._a, self._g, _abi._fptr(ckpt.data_ptr()), ckpt.numel() * 4)
        self._fn = getattr(_abi.load(), self.func)

    def launch(self, stream=None):
        if stream is None:
            stream = torch.cuda.current_stream(self.device).cuda_stream
        st = self._fn(*self._refs, _abi._vp(stream))
        if st != _abi.R2L_OK:
            raise R2LError(st, self.func, _abi.last_error())


def bind_backward(x, dt, Bm, Cm, A, Dskip=None, *, dout, **kw) -> BoundBackward:
    """Check and marshal a ``r2l_scan_backward`` call once (same keywords);
    the outputs are allocated here (or taken from ``out``)."""
    kw = dict(kw)
    kw["_bind"] = True
    return r2l_scan_backward(x, dt, Bm, Cm, A, Dskip, dout=dout, **kw)


def prefix_scan_backward(x, dt, Bm, Cm, A, Dskip=None, **kw):
    """Gradients of ``prefix_scan_state`` with readout (``Cm``, residual and
    out: the left-to-right stream), same keywords as ``r2l_scan_backward``."""
    return r2l_scan_backward(x, dt, Bm, Cm, A, Dskip, _reverse=False, **kw)


def r2l_scan_backward(x, dt, Bm, Cm, A, Dskip=None, *, dout, dh_out=None, cu_seqlens=None,
                      max_seqlen=None, h_in=None, res=None, s=0.0, delta_softplus=True,
                      grads=GRADS, out=None, workspace=None, chunk_tokens=0, ckpt=None,
                      _bind=False, _reverse=True):
    """Gradients of ``r2l_scan`` (same forward arguments) for ``dout`` = dL/dout
    and ``dh_out`` = dL/dh_out. Returns a dict of the names in ``grads``: dx,
    ddt (like x), dBm, dCm (fp32, shaped like Bm), dA [D, N], dDskip [D],
    dh_in [batch, D, N], ds [1] (with a residual only). ``out`` may hold
    preallocated tensors for some of them. A separate residual's gradient is
    dout itself; when res is x, dx includes it. ``chunk_tokens`` is the
    planning hint of the backward's state pass (0: the library chooses).
    ``ckpt``: the checkpoints ``r2l_scan_save`` stored for the same forward
    arguments; the backward then runs no forward state pass."""
    if ckpt is not None and (ckpt.dtype != torch.float32 or not ckpt.is_contiguous()):
        raise ValueError("ckpt must be a contiguous fp32 tensor")
    a = _fill(x, dt, Bm, Cm, A, Dskip, cu_seqlens, max_seqlen, h_in, None, res, s, None,
              delta_softplus, chunk_tokens, 0)
    D, N = int(a.dim), int(a.dstate)
    outs = dict(out or {})
    wanted = [n for n in grads if n != "ds" or res is not None]
    make = {"dx": lambda: torch.empty_like(x), "ddt": lambda: torch.empty_like(x),
            "dBm": lambda: torch.empty(Bm.shape, dtype=torch.float32, device=x.device),
            "dCm": lambda: torch.empty(Bm.shape, dtype=torch.float32, device=x.device),
            "dA": lambda: torch.empty((D, N), dtype=torch.float32, device=x.device),
            "dDskip": lambda: torch.empty((D,), dtype=torch.float32, device=x.device),
            "dh_in": lambda: torch.empty((a.batch, D, N), dtype=torch.float32, device=x.device),
            "ds": lambda: torch.empty((1,), dtype=torch.float32, device=x.device)}
    for n in wanted:
        if outs.get(n) is None:
            outs[n] = make[n]()
    outs = {n: outs[n] for n in wanted}
    g = _fill_grad(a, x, Bm, dout, dh_out, outs)
    need = _abi.backward_workspace_size(a, g)
    if need:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
        elif workspace.numel() * workspace.element_size() < need:
            raise ValueError("workspace has %d bytes, the backward needs %d"
                             % (workspace.numel() * workspace.element_size(), need))
        g.workspace, g.workspace_bytes = workspace.data_ptr(), need
    if _bind:
        keep = (x, dt, Bm, Cm, A, Dskip, dout, dh_out, cu_seqlens, h_in, res)
        return BoundBackward(a, g, keep, outs, workspace, x.device, reverse=_reverse, ckpt=ckpt)
    with torch.cuda.device(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
    if ckpt is not None:
        _abi.call_backward_saved(a, g, ckpt.data_ptr(), ckpt.numel() * 4, stream, reverse=_reverse)
    else:
        _abi.call_backward(a, g, stream, reverse=_reverse)
    return outs


class R2LScan(torch.autograd.Function):
    """The R2L stream as a differentiable op (dense [batch, L, D] tensors):
    out = x + s * y (the hook) or y (``s`` None). ``s`` is a float (a fixed
    gate) or a one-element fp32 tensor (the learnable gate, initialised at
    zero, which receives ds = sum(dout * y); its value is read on the host for
    the call). Gradients flow to x, dt, Bm, Cm, A and Dskip (and s) through
    ``r2l_scan_backward``: from the state checkpoints that the forward
    (``r2l_scan_save``) stored when any of x..Dskip needs a gradient, else
    through the backward's own state pass."""

    @staticmethod
    def forward(ctx, x, dt, Bm, Cm, A, Dskip, s=None):
        res = x if s is not None else None
        s_tensor = isinstance(s, torch.Tensor)
        if s_tensor and s.numel() != 1:
            raise ValueError("s must be a float or a one-element tensor")
        gate = 0.0 if s is None else float(s.item() if s_tensor else s)
        if any(ctx.needs_input_grad[:6]):
            out, ckpt = r2l_scan_save(x, dt, Bm, Cm, A, Dskip, res=res, s=gate)
        else:   # no checkpoints: a gradient of s alone runs the backward's state pass
            out, ckpt = r2l_scan(x, dt, Bm, Cm, A, Dskip, res=res, s=gate), None
        ctx.save_for_backward(x, dt, Bm, Cm, A, Dskip, ckpt)
        ctx.gate, ctx.has_res, ctx.s_tensor = gate, s is not None, s_tensor
        ctx.s_like = (s.shape, s.dtype) if s_tensor else None
        return out

    @staticmethod
    def backward(ctx, dout):
        x, dt, Bm, Cm, A, Dskip, ckpt = ctx.saved_tensors
        want_ds = ctx.s_tensor and ctx.needs_input_grad[6]
        names = ("dx", "ddt", "dBm", "dCm", "dA", "dDskip") + (("ds",) if want_ds else ())
        g = r2l_scan_backward(x, dt, Bm, Cm, A, Dskip, dout=dout.contiguous(),
                              res=x if ctx.has_res else None, s=ctx.gate, ckpt=ckpt, grads=names)
        ds = g["ds"].reshape(ctx.s_like[0]).to(ctx.s_like[1]) if want_ds else None
        return (g["dx"], g["ddt"], g["dBm"].to(Bm.dtype), g["dCm"].to(Cm.dtype), g["dA"],
                g["dDskip"] if Dskip is not None else None, ds)